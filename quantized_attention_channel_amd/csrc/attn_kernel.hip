// Fused quantised attention forward for gfx950.
//
// One work-group = 8 waves = two groups of 4, each group one 128-query tile of
// the same (batch, query head); each wave owns 32 queries and walks the KV
// sequence in tiles of 128 keys, which all eight waves share through LDS
// (double-buffered). The two groups run half a tile apart so that the matrix
// work of one overlaps the vector work of the other (see the kernel below).
//
// Per wave and tile (SageAttention's hot loop: INT8 QK^T, online softmax, P in
// FP8 or FP16, PV with two-level accumulation -- thu-ml/SageAttention repo card,
// "How it works"; heatdrop.ai review, "The interesting bit"):
//   1. S^T[128 keys x 32 queries] = K8 . Q8^T on the INT8 matrix cores (INT32
//      accumulation), as four 32-key blocks. Computing the transpose puts one
//      query per lane: lane l holds query l % 32 and 16 keys of every block, so
//      each row reduction is in-lane plus one exchange with lane l ^ 32.
//   2. Dequantise with c = s_q * s_k * sm_scale * log2(e) (per-block scales:
//      one factor per 64-key K block, a group being one Q block; per-thread
//      scales: the lane's own query and each 16 keys the lane holds), mask only
//      on the causal diagonal / ragged tail tile, online softmax in the log2
//      domain.
//   3. P -> e4m3 (scaled by 448 through the exponent) or fp16/bf16, packed
//      straight from registers into the B operand of the PV product: the K rows
//      of step 1 are permuted so that each lane's keys are contiguous, exactly
//      the key order the PV operand needs.
//   4. PV with two-level accumulation: each matrix instruction sums the
//      products of its 64 (FP8) or 16 (FP16/BF16) keys (level 1) into the fp32
//      accumulator O (level 2), after O = alpha * O when a row's max moved.
// Epilogue: O * s_v[c] / l (FP8) or O / l, rounded to the input dtype and
// stored in the caller's layout.
#include <climits>
#include <type_traits>

#include "attn_schedule.h"
#include "sage_device.h"
#include "sage_launch.h"

#ifndef SAGE_PHASE_TRACE
#define SAGE_PHASE_TRACE 0   // 1: the diagnostic per-phase cycle trace build (phase_trace.py)
#endif

namespace sage {

constexpr int kBq = 128;           // queries per group == the Q quantisation block
constexpr int kBlocks = kBkv / 32; // 32-key S^T blocks per tile
static_assert(kBkv == 2 * kBlkK, "a tile spans two K quantisation blocks");
static_assert(kFineBlkK == 16 && kFineBlkQ == 1, "per-thread scales follow the lane layout of the products");

// --------------------------------------------------------------- LDS layouts
// gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a time from 64 banks
// (256 bytes per cycle); a read is conflict-free when every group of 16
// consecutive lanes covers the 16 distinct 16-byte slots of a 256-byte span.
// Each layout XOR-swizzles the 16-byte chunk index with bits of the row so the
// operand reads of the kernel below meet that rule.
//
// K tile: [128 keys][D bytes]. A lane group reads 16 rows key_perm(0..15)
// (+16) of one chunk column; the swizzle uses the row bits that vary among them.
template <int D>
__device__ __forceinline__ int key_swz(int row) {
  if constexpr (D == 128) return ((row >> 1) & 3) | (((row >> 4) & 1) << 2);   // 8 chunks per row
  else return ((row >> 2) & 1) | (((row >> 4) & 1) << 1);                      // 4 chunks per row
}
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  return row * D + ((chunk ^ key_swz<D>(row)) << 4);
}
// A row m of a 32-key block reads key key_perm(m); the S^T result then holds
// keys 16*g .. 16*g+15 of the block in lane group g, in element order.
__device__ __forceinline__ int key_perm(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }
// V^T tile: [D channels][128 keys] of 1 (e4m3: 8 chunks per row) or 2
// (fp16/bf16: 16 chunks per row) bytes per key; a lane group reads 16
// consecutive rows of one chunk column.
template <bool FP8>
__device__ __forceinline__ int v_swz(int row) { return FP8 ? ((row >> 1) & 7) : (row & 15); }
template <bool FP8>
__device__ __forceinline__ int v_lds_off(int row, int chunk) {
  constexpr int rowb = FP8 ? kBkv : 2 * kBkv;
  return row * rowb + ((chunk ^ v_swz<FP8>(row)) << 4);
}

__device__ __forceinline__ i32x4 lds16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }

// --------------------------------------------------------------- tile staging
// Direct global -> LDS loads (no staging registers): in each wave-wide load,
// lane L writes 16 bytes at LDS slot base + 16 * L, so every lane fetches the
// global chunk that the swizzled layout puts in its slot. Per-lane offsets do
// not depend on the tile. The buffer range check covers only the per-lane
// (VGPR) offset, not the scalar one, so each K load pass gets its own resource,
// based at the pass's first byte and sized to the bytes of the head that
// remain: K rows past Nk then read as zeros and no load leaves the K slice.
// V^T rows are padded to whole tiles, so every V load lies inside its rows and
// the tile offset can ride in the scalar offset.
template <int D, bool FP8, int NW>
struct TileStage {
  static constexpr int kVRowB = kBkv * (FP8 ? 1 : 2);
  static constexpr int kPass = NW * 1024;                // LDS bytes per wave-wide load pass
  static constexpr int kKLoads = kBkv * D / kPass;       // load passes per tile
  static constexpr int kVLoads = D * kVRowB / kPass;
  static constexpr int kEb = FP8 ? 1 : 2;
  // Load pass i covers LDS bytes [kPass i, kPass (i+1)) of a tile: K rows
  // kPass/D apart, V^T rows kPass/kVRowB apart. Both swizzles read only row
  // bits below those strides, so pass i's global offsets are pass 0's plus
  // a constant, which goes in the scalar offset: one VGPR per tensor.
  static constexpr int kVRowsPerPass = kPass / kVRowB;
  static_assert(kKLoads >= 1 && kVLoads >= 1, "every wave loads");
  static_assert(kPass / D >= 32 && kVRowsPerPass >= 16, "swizzle bits stay below the pass stride");

  static __device__ __forceinline__ uint32_t init_k(int wave, int lane) {
    const int slot = wave * 64 + lane;                    // pass 0
    const int krow = slot / (D / 16), kchunk = slot % (D / 16);
    return (uint32_t)krow * D + ((kchunk ^ key_swz<D>(krow)) << 4);
  }
  static __device__ __forceinline__ void init(uint32_t& koff, uint32_t& voff, int wave, int lane, int n_pad) {
    const int slot = wave * 64 + lane;                    // pass 0
    koff = init_k(wave, lane);
    const int vrow = slot / (kVRowB / 16), vchunk = slot % (kVRowB / 16);
    voff = (uint32_t)vrow * n_pad * kEb + ((vchunk ^ v_swz<FP8>(vrow)) << 4);
  }
  // kbase/kbytes: this head's K codes [Nk][D] (or a packed sequence's)
  static __device__ __forceinline__ void issue_k(const int8_t* kbase, uint32_t kbytes, uint32_t koff, int wave,
                                                 int k0, int8_t* sk) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const uint32_t start = __builtin_amdgcn_readfirstlane((uint32_t)k0 * D + i * kPass);
      const auto rk = make_rsrc(kbase + start, tail_bytes(kbytes, start));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(sk + (i * NW + wave) * 1024),
                                              16, koff, 0, 0, 0);
    }
  }
  static __device__ __forceinline__ void issue_k_pass(const int8_t* kbase, uint32_t kbytes, uint32_t koff, int wave,
                                                      int k0, int8_t* sk, int i) {
    const uint32_t start = __builtin_amdgcn_readfirstlane((uint32_t)k0 * D + i * kPass);
    const auto rk = make_rsrc(kbase + start, tail_bytes(kbytes, start));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(sk + (i * NW + wave) * 1024),
                                            16, koff, 0, 0, 0);
  }
  static __device__ __forceinline__ void issue_v_pass(__amdgpu_buffer_rsrc_t rv, uint32_t voff, int wave, int k0,
                                                      int n_pad, uint8_t* sv, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(sv + (i * NW + wave) * 1024),
                                            16, voff, (k0 + i * kVRowsPerPass * n_pad) * kEb, 0, 0);
  }
  // rv covers this head's V^T rows [D][n_pad]
  static __device__ __forceinline__ void issue_v(__amdgpu_buffer_rsrc_t rv, uint32_t voff, int wave, int k0,
                                                 int n_pad, uint8_t* sv) {
#pragma unroll
    for (int i = 0; i < kVLoads; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(sv + (i * NW + wave) * 1024),
                                              16, voff, (k0 + i * kVRowsPerPass * n_pad) * kEb, 0, 0);
  }
};

// Scores as floats without a conversion instruction. For any INT8 codes
// (-128 included) |S| <= D * 128 * 128 < 2^22 at D <= 128, so the integer
// kScoreOffset + S is the fp32 bit pattern of the float kScoreOffsetF + S
// exactly (floats in [2^23, 2^24] are the integers there), and one exact
// subtraction gives float(S). The product chain adds the offset
// for free when it starts from it instead of zero; the integer order of the
// offset codes is that of S, so the row maximum still runs on integers.
constexpr int kScoreOffset = 0x4B400000;
constexpr float kScoreOffsetF = 12582912.0f;   // 1.5 * 2^23
static_assert(128 * 128 * 128 < (1 << 22), "scores of the largest head dimension stay inside the offset binade");
__device__ __forceinline__ float as_f32(int v) { return __builtin_bit_cast(float, v); }

// S^T for the 128 keys of the staged tile against this wave's 32 queries.
// Every product chain starts from c0: zero gives S itself, kScoreOffset in
// every element gives the fp32 bit patterns of kScoreOffsetF + S.
template <int D>
__device__ __forceinline__ void qk_tile(const int8_t* sk, const i32x4* qreg, int lane, i32x16* s, const i32x16& c0) {
  const int g = lane >> 5, m = lane & 31;
  const int r0 = key_perm(m);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      const i32x4 ka = lds16(sk + k_lds_off<D>(32 * b + r0, 2 * t + g));
      s[b] = mfma_i8(ka, qreg[t], t == 0 ? c0 : s[b]);
    }
    if (t % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // at most 8 K operands in flight
  }
}

template <int D>
__device__ __forceinline__ void load_q_operand(const int8_t* q8_head, int nq, int qi, int g, i32x4* qreg) {
  const auto rq = make_rsrc(q8_head, (uint32_t)nq * D);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) qreg[t] = buf_load16(rq, (uint32_t)qi * D + 32 * t + 16 * g);
}

// Per-wave online-softmax state and the fp32 output accumulator (level 2).
template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m;
  float l;
};

template <typename T>
using Half8 = typename std::conditional<std::is_same<T, BF16>::value, bf16x8, f16x8>::type;

// P of one tile as the PV product consumes it, with the tile's rescale factor.
template <bool FP8, typename T>
struct PTile;
template <typename T>
struct PTile<true, T> {
  i32x8 pk[2];       // e4m3 codes of 448 P~; pk[u]: key half u (bytes 0..15 block 2u, 16..31 block 2u+1)
  float alpha;
};
template <typename T>
struct PTile<false, T> {
  Half8<T> ph[2 * kBlocks];   // ph[2b + h]: block b, keys 16g + 8h + 0..7
  float alpha;
  float lsum;                 // this lane's sum of the rounded P
};

// Softmax phase of one KV tile for one wave (vector ALU work only): mask,
// online softmax in the log2 domain, P quantisation. s (S^T of the tile) is
// consumed; the running max is updated; the P operand and alpha go to pt.
// c[bb]: this lane's dequantisation factor for 32-key block bb (per-block
// scales: one per 64-key half of the tile; per-thread: one per lane half).
template <int D, bool FP8, bool CAUSAL, bool MASK, bool FINE, typename T>
__device__ __forceinline__ void softmax_phase(i32x16* s, int lane, int k0, int qi, int nk, const float (&c)[kBlocks],
                                              float& m, PTile<FP8, T>& pt) {
  const int g = lane >> 5;
  if (MASK) {
    // key k0 + 32b + 16g + r is visible iff 32b + r < lim (one per-lane bound
    // against compile-time constants)
    const int lim = (CAUSAL ? min(nk, qi + 1) : nk) - k0 - 16 * g;
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * bb + r >= lim) s[bb][r] = INT_MIN;
  }
  // Row maximum per K quantisation block: four chains of one 3-input integer
  // max per two scores (the pins keep the compiler from rebalancing them into
  // a tree of 2-input maxima), then scaled.
  auto si = [&](int bb, int r) { const int v = s[bb][r]; return v; };
  int mc[kBlocks] = {si(0, 0), si(1, 0), si(2, 0), si(3, 0)};
#pragma unroll
  for (int r = 1; r < 15; r += 2)
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb) {
      mc[bb] = max(mc[bb], max(si(bb, r), si(bb, r + 1)));
      pin(mc[bb]);
    }
  // (FP8 P: the scores carry kScoreOffset; FP16 P keeps plain S and the
  //  conversion, since the 16 registers of the offset block do not fit there)
  auto sf = [&](int v) { return FP8 ? as_f32(v) - kScoreOffsetF : (float)v; };
  float m_tile;
  if constexpr (FINE) {
    float tb[kBlocks];
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb) {
      const int mxb = max(mc[bb], si(bb, 15));
      tb[bb] = sf(mxb) * c[bb];
      if (MASK && mxb == INT_MIN) tb[bb] = -INFINITY;
    }
    m_tile = fmaxf(fmaxf(tb[0], tb[1]), fmaxf(tb[2], tb[3]));
  } else {
    const int mx0 = max(max(mc[0], si(0, 15)), max(mc[1], si(1, 15)));
    const int mx1 = max(max(mc[2], si(2, 15)), max(mc[3], si(3, 15)));
    float t0 = sf(mx0) * c[0], t1 = sf(mx1) * c[2];
    if (MASK) {
      if (mx0 == INT_MIN) t0 = -INFINITY;
      if (mx1 == INT_MIN) t1 = -INFINITY;
    }
    m_tile = fmaxf(t0, t1);
  }
  const float m_new = fmaxf(m, pair_max(m_tile));
  pt.alpha = fast_exp2(m - m_new);
  m = m_new;
  const float bias = (FP8 ? kLog2E4m3Max : 0.0f) - m_new;   // P8 = e4m3(448 * P~) via the exponent

  // P~ overwrites the scores in place (as fp32 bit patterns).
#pragma unroll
  for (int bb = 0; bb < kBlocks; ++bb) {
    const float cb = FINE ? c[bb] : c[bb < 2 ? 0 : 2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int sv = si(bb, r);
      float x = fast_exp2(__builtin_fmaf(sf(sv), cb, bias));
      if (MASK && sv == INT_MIN) x = 0.0f;
      s[bb][r] = __builtin_bit_cast(int, x);
    }
  }
  // (copy the element out first: a bit-cast applied to a vector-element
  //  expression reads the vector's first element)
  auto p = [&](int bb, int r) { const int bits = s[bb][r]; return __builtin_bit_cast(float, bits); };
  // The first conversion of each pair writes the low half and keeps the high
  // half of its third operand, which the second conversion overwrites: any
  // value serves, and reusing an input's register avoids initialising one.
  auto bits = [&](int bb, int r) { const int v = s[bb][r]; return v; };
  if constexpr (FP8) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p(2 * u, 4 * w), p(2 * u, 4 * w + 1), bits(2 * u, 4 * w), false);
        pt.pk[u][w] = __builtin_amdgcn_cvt_pk_fp8_f32(p(2 * u, 4 * w + 2), p(2 * u, 4 * w + 3), x, true);
        int y = __builtin_amdgcn_cvt_pk_fp8_f32(p(2 * u + 1, 4 * w), p(2 * u + 1, 4 * w + 1), bits(2 * u + 1, 4 * w),
                                                false);
        pt.pk[u][4 + w] = __builtin_amdgcn_cvt_pk_fp8_f32(p(2 * u + 1, 4 * w + 2), p(2 * u + 1, 4 * w + 3), y, true);
      }
  } else {
    using HS = typename std::conditional<std::is_same<T, BF16>::value, __bf16, _Float16>::type;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pt.ph[2 * b][e] = (HS)p(b, e);
        pt.ph[2 * b + 1][e] = (HS)p(b, 8 + e);
      }
    // Row sum of the rounded P (the values the PV product consumes), two per
    // dot instruction; each lane holds its half of the keys.
    float lsum = 0.0f;
#pragma unroll
    for (int u = 0; u < 2 * kBlocks; ++u)
#pragma unroll
      for (int e = 0; e < 8; e += 2) lsum = dot2_ones(pt.ph[u][e], pt.ph[u][e + 1], lsum);
    pt.lsum = lsum;
  }
  if constexpr (FP8) {
    pin(pt.pk[0]);
    pin(pt.pk[1]);
  } else {
#pragma unroll
    for (int u = 0; u < 2 * kBlocks; ++u) pin(pt.ph[u]);
    pin(pt.lsum);
  }
  pin(pt.alpha);
  pin(m);
}

// PV phase of one KV tile for one wave (matrix-core work): the row sum of the
// quantised P, then O = alpha O + V^T P^T. Level 1 of the accumulation is the
// sum of one matrix instruction's products (64 keys in FP8, 16 in FP16/BF16),
// level 2 the fp32 accumulator O that each instruction adds its sum into. The
// rescale by alpha runs only when some row of the wave raised its maximum
// (alpha != 1); with long sequences most tiles leave every row's max alone,
// and the 16 multiplies per channel block are then skipped.
// O = alpha O before a tile's products are added, skipped when alpha is 1 on
// every lane (a wave-uniform branch: exp2(0) is exactly 1, so a row whose
// maximum did not move keeps O unchanged either way).
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

template <int D, bool FP8, typename T, typename Hook = NoHook>
__device__ __forceinline__ void pv_phase(const uint8_t* sv, int lane, const PTile<FP8, T>& pt, RowState<D>& st,
                                         const Hook& hook = Hook{}) {
  constexpr int NT = D / 32;
  const int g = lane >> 5, n = lane & 31;
  const float alpha = pt.alpha;
  if constexpr (FP8) {
    // V^T operands of 32-channel block cb: rows cb*32 + n, 16-byte chunks
    // 4u + g and 4u + 2 + g for key half u. Read one block ahead of its MFMAs.
    auto load_v = [&](int cb, i32x8* va) {
      const int row = cb * 32 + n;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const i32x4 lo = lds16(sv + v_lds_off<true>(row, 4 * u + g));
        const i32x4 hi = lds16(sv + v_lds_off<true>(row, 4 * u + 2 + g));
        va[u] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    i32x8 va[NT][2];
    load_v(0, va[0]);
    // Row sum of the quantised P (the values the PV product consumes): with an
    // all-ones A operand every row of the product is the sum over the tile's
    // keys, so each lane receives its query's complete sum.
    {
      constexpr int kOnes = 0x38383838;                 // four e4m3 1.0
      const i32x8 ones = {kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};
      f32x16 ls = mfma_fp8(ones, pt.pk[0], f32x16{});
      ls = mfma_fp8(ones, pt.pk[1], ls);
      st.l = __builtin_fmaf(alpha, st.l, ls[0]);
    }
    rescale_o<D>(alpha, st);
#pragma unroll
    for (int cb = 0; cb < NT; ++cb) {
      if (cb + 1 < NT) load_v(cb + 1, va[cb + 1]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        st.o[cb] = mfma_fp8(va[cb][u], pt.pk[u], st.o[cb]);
        hook(2 * cb + u);
      }
    }
  } else {
    using H8 = Half8<T>;
    st.l = __builtin_fmaf(alpha, st.l, pt.lsum);
    rescale_o<D>(alpha, st);
#pragma unroll
    for (int cb = 0; cb < NT; ++cb) {
      const int row = cb * 32 + n;
#pragma unroll
      for (int u = 0; u < 2 * kBlocks; ++u) {
        // keys 32*(u/2) + 16g + 8*(u%2) + 0..7 -> 16-byte chunk 4*(u/2) + 2g + (u%2)
        const i32x4 raw = lds16(sv + v_lds_off<false>(row, 4 * (u >> 1) + 2 * g + (u & 1)));
        st.o[cb] = mfma_half(__builtin_bit_cast(H8, raw), pt.ph[u], st.o[cb]);
        hook(2 * kBlocks * cb + u);
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < NT; ++cb) pin(st.o[cb]);
  pin(st.l);
}

// --------------------------------------------------------------- the kernel
// One work-group = 8 waves = two groups of four, each group one 128-query tile
// (one Q quantisation block) of the same (batch, head); each wave owns 32
// queries. The groups share the K/V tiles in LDS and run half a tile apart
// ("ping-pong"): while one group is in its matrix phase (PV of the previous
// tile, then QK^T of this one) the other is in its vector phase (softmax of its
// current tile), so on every SIMD one wave keeps the matrix cores busy while
// the other issues vector instructions. Every phase ends at a work-group
// barrier.
//
// Global phase p: group 0 runs X(t) at p = 2t and Y(t) at p = 2t + 1; group 1
// runs one phase later. X(t) = PV(t-1) + QK^T(t), Y(t) = softmax(t). K(t) is
// read in phases 2t and 2t+1, V(t-1) in the same two phases. Group 0 issues
// the load of K(t+1) in phase 2t (into the buffer K(t-1) left), group 1 the
// load of V(t) in phase 2t+1 (into the buffer V(t-2) left), each during its
// matrix phase; both must land by the end of phase 2t+1.
constexpr int kWaves = 8;


template <int D, bool FP8, bool CAUSAL, typename T, bool FINE>
__device__ __forceinline__ void attn_fwd_body(AttnArgs a) {
  constexpr int NT = D / 32;
  using Stage = TileStage<D, FP8, kWaves>;
  constexpr int kKBytes = kBkv * D, kVBytes = D * Stage::kVRowB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kKBytes + 2 * kVBytes];
#if SAGE_PHASE_TRACE >= 2
  const uint64_t tr_entry = __builtin_readcyclecounter();
  const uint64_t rt_entry = __builtin_amdgcn_s_memrealtime();
#endif

  // Work decomposition. Work-groups are dealt round-robin to the 8 XCDs; give
  // each XCD a contiguous range of (head, query) work so the work-groups that
  // share an XCD's L2 stream the same head's K/V tiles.
  //   Packed variable-length batches: the sequences' work differs widely, so
  // contiguous (sequence, head) ranges would load some XCDs several times more
  // than others. There XCD x takes heads [x Hq/8, (x+1) Hq/8) of every sequence
  // (when Hq % 8 == 0; else plain round-robin) and walks the work list of
  // query pairs: sequence by sequence, each sequence's pairs from the last
  // (longest under causal masking) down, the heads of one pair side by side.
  // The work-groups running together then share one sequence's K/V tiles in
  // the XCD's L2, and no work-group is spent on pairs a sequence lacks.
  const int n_qp = (a.Nq + 2 * kBq - 1) / (2 * kBq);
  int bh, qp;
  if (a.seq) {
    int heads = a.Hq, h0 = 0, j = blockIdx.x;
    if ((a.Hq & 7) == 0) {
      heads = a.Hq >> 3;
      h0 = (blockIdx.x & 7) * heads;
      j = blockIdx.x >> 3;
    }
    const int qpi = j / heads;                                   // work-list query pair
    const int sb = qpi < a.n_owner ? a.qp_owner[qpi] : -1;
    if (sb < 0) return;                                          // past the work list
    qp = (a.seq[sb].nq + 2 * kBq - 1) / (2 * kBq) - 1 - (qpi - a.seq[sb].qp0);
    bh = sb * a.Hq + h0 + j % heads;
  } else {
    const int total = n_qp * a.B * a.Hq;
    int id = blockIdx.x;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
    bh = id / n_qp;
    qp = id % n_qp;
    if (CAUSAL) qp = n_qp - 1 - qp;            // longest rows first
  }
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int bhk = b * a.Hkv + hk;

  // This work-group's query and key ranges: the whole batch entry, or (packed
  // variable-length batch) its sequence's ranges from the span table, with the
  // codes stored [H][total][D] and V^T in the sequence's columns of the rows.
  int nq = a.Nq, nk = a.Nk;
  int64_t q_off = (int64_t)bh * a.Nq * D, k_off = (int64_t)bhk * a.Nk * D;
  int64_t v_off = (int64_t)bhk * D * a.n_pad, v_len = (int64_t)D * a.n_pad, o_tok = 0;
  if (a.seq) {
    const SeqSpan sp = a.seq[b];
    nq = sp.nq;
    nk = sp.nk;
    if (2 * qp * kBq >= nq) return;              // no rows of this sequence here
    q_off = ((int64_t)h * a.total_q + sp.q0) * D;
    k_off = ((int64_t)hk * a.total_k + sp.k0) * D;
    v_off = (int64_t)hk * D * a.n_pad + sp.kp0;
    v_len = (int64_t)D * a.n_pad - sp.kp0;
    o_tok = sp.q0;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int g = lane >> 5;
  const int qt = 2 * qp + grp;                 // this group's 128-query tile
  const int q0w = qt * kBq + (wave & 3) * 32;
  const int qi = q0w + (lane & 31);

  i32x4 qreg[NT];
  load_q_operand<D>(a.q8 + q_off, nq, qi, g, qreg);
  const bool grp_live = qt * kBq < nq;
  // Q scale: the group's block, or (per-thread) the lane's own query.
  float cq;
  if constexpr (FINE) cq = qi < nq ? a.q_scale[(int64_t)bh * a.nbq + qi] * a.scale_log2 : 0.0f;
  else cq = grp_live ? a.q_scale[(int64_t)bh * a.nbq + qt] * a.scale_log2 : 0.0f;
  const __attribute__((address_space(4))) float* kscale =
      (const __attribute__((address_space(4))) float*)(a.k_scale + (int64_t)bhk * a.nbk);

  // KV tiles this group attends to, and the work-group's (the longer of the two).
  // Only a group's last tile can need masking: it holds the ragged end of the
  // keys and, with causal masking (Nq == Nk, query tile == KV tile), the diagonal.
  auto tiles_for = [&](int q_tile) {
    const int kv_end = CAUSAL ? min(nk, (q_tile + 1) * kBq) : nk;
    return (kv_end + kBkv - 1) / kBkv;
  };
  const int n_g = grp_live ? tiles_for(qt) : 0;
  const int n_wg = ((2 * qp + 1) * kBq < nq) ? tiles_for(2 * qp + 1) : tiles_for(2 * qp);

  constexpr int eb = FP8 ? 1 : 2;
  const int8_t* kbase = a.k8 + k_off;
  const uint32_t kbytes = (uint32_t)nk * D;
  const auto rv = make_rsrc(reinterpret_cast<const uint8_t*>(a.vt) + v_off * eb, (uint32_t)(v_len * eb));
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // All eight waves load the first K tile.
  const uint32_t koff = Stage::init_k(wv, lane);
  // After the first tile, group 0's four waves load each pair's tiles, at the
  // end of their matrix phase (before it in the last two pairs, where the
  // buffer parity is known only at run time). That phase ends before group 1's
  // softmax phase, so the wait for the address unit to take the loads falls
  // into time group 0 would spend at the barrier, and no other wave issues
  // loads.
  using StageG = TileStage<D, FP8, 4>;
  uint32_t koffg, voffg;
  StageG::init(koffg, voffg, wv & 3, lane, a.n_pad);
  Stage::issue_k(kbase, kbytes, koff, wv, 0, reinterpret_cast<int8_t*>(smem));
  wait_loads_barrier();

  RowState<D> st;
#pragma unroll
  for (int cb = 0; cb < NT; ++cb) st.o[cb] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.0f;

  // Buffers by tile parity, as compile-time offsets: the compiler can then tell
  // the buffer being loaded from the one being read, and does not wait for a
  // prefetch before an unrelated LDS read.
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  i32x16 s[kBlocks];
  PTile<FP8, T> pt;
  // The start value of every QK^T chain, kept in registers (opaque, so that
  // it is not rebuilt per tile): the score offset for FP8 P, else zero.
  i32x16 qk_init;
#pragma unroll
  for (int e = 0; e < 16; ++e) qk_init[e] = FP8 ? kScoreOffset : 0;
  if constexpr (FP8) pin(qk_init);

  // Phase pair t = global phases 2t and 2t+1, P = t & 1. The tile loads are
  // split between the groups, each issuing its share while its own matrix
  // work runs: group 0 loads K(t+1) in phase 2t (into the buffer K(t-1)
  // left), group 1 loads V(t) in phase 2t+1 (into the buffer V(t-2) left).
  // Both land by the wait that ends the pair. A load instruction holds its
  // wave until the address unit takes it (about one matrix instruction's
  // time per kilobyte and wave when four waves load together), so one group
  // carrying all of them lengthened its matrix phase past the other group's
  // softmax phase; split, each matrix phase takes half and the two phases of
  // a pair balance.
  auto loads_k = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    if (t + 1 < n_wg)
      StageG::issue_k(kbase, kbytes, koffg, wv & 3, (t + 1) * kBkv, reinterpret_cast<int8_t*>(smem + (1 - P) * kKBytes));
  };
  auto loads_v = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    if (t < n_wg) StageG::issue_v(rv, voffg, wv & 3, t * kBkv, a.n_pad, smem + 2 * kKBytes + P * kVBytes);
  };
  // (the last pairs and the idle pairs: runtime parity)
  auto loads_k_rt = [&](int t) __attribute__((always_inline)) {
    if (t & 1) loads_k(Odd{}, t); else loads_k(Even{}, t);
  };
  auto loads_v_rt = [&](int t) __attribute__((always_inline)) {
    if (t & 1) loads_v(Odd{}, t); else loads_v(Even{}, t);
  };
  // X(t): PV(t-1) with V in buffer 1-P, then QK^T(t) with K in buffer P.
  auto x_bufs = [&](const uint8_t* v_prv, const int8_t* k_cur, bool do_pv, bool do_qk,
                    const auto& hook) __attribute__((always_inline)) {
    // The matrix wave outranks the softmax wave while it issues PV (and the
    // rescale of O, when taken), which must not wait behind the softmax's
    // exps; its QK^T part competes at equal priority.
    __builtin_amdgcn_s_setprio(1);
    if (do_pv) pv_phase<D, FP8, T>(v_prv, lane, pt, st, hook);
    __builtin_amdgcn_sched_barrier(0);         // P and the V operands die before the K operands load
    __builtin_amdgcn_s_setprio(0);
    if (do_qk) qk_tile<D>(k_cur, qreg, lane, s, qk_init);
  };
  auto x_phase = [&](auto par, int t, bool do_pv, bool do_qk) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    x_bufs(smem + 2 * kKBytes + (1 - P) * kVBytes, reinterpret_cast<const int8_t*>(smem + P * kKBytes), do_pv, do_qk,
           NoHook{});
  };
  // X(t) in the steady pairs with this group's loads issued one after each
  // PV product, so that the wait for the address unit overlaps matrix work
  // already issued: K(t+1) for group 0, V(t) for group 1.
  auto x_phase_loading = [&](auto par, int t) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    int8_t* kdst = reinterpret_cast<int8_t*>(smem + (1 - P) * kKBytes);
    uint8_t* vdst = smem + 2 * kKBytes + P * kVBytes;
    auto hook = [&](int j) __attribute__((always_inline)) {
      if (grp == 0) {
        if (j < StageG::kKLoads && t + 1 < n_wg)
          StageG::issue_k_pass(kbase, kbytes, koffg, wv & 3, (t + 1) * kBkv, kdst, j);
      } else {
        if (j < StageG::kVLoads && t < n_wg) StageG::issue_v_pass(rv, voffg, wv & 3, t * kBkv, a.n_pad, vdst, j);
      }
    };
    x_bufs(smem + 2 * kKBytes + (1 - P) * kVBytes, reinterpret_cast<const int8_t*>(smem + P * kKBytes), true, true,
           hook);
  };
  // The same with the parity known only at run time (the last pairs of a
  // group): the compiler then cannot separate these reads from the prefetch in
  // flight and waits for it first, which costs a load latency once or twice
  // per work-group.
  auto x_phase_rt = [&](int t, bool do_pv, bool do_qk) __attribute__((always_inline)) {
    const int P = t & 1;
    x_bufs(smem + 2 * kKBytes + (1 - P) * kVBytes, reinterpret_cast<const int8_t*>(smem + P * kKBytes), do_pv, do_qk,
           NoHook{});
  };
  // Y(t): softmax of tile t (registers only).
  auto y_phase = [&](int t, auto masked) __attribute__((always_inline)) {
    float c[kBlocks];
    if constexpr (FINE) {
      // lane half g holds keys 32bb + 16g + 0..15 of the tile: scale 8t + 2bb + g
#pragma unroll
      for (int bb = 0; bb < kBlocks; ++bb) {
        const float ka = kscale[min(8 * t + 2 * bb, a.nbk - 1)];
        const float kb = kscale[min(8 * t + 2 * bb + 1, a.nbk - 1)];   // past Nk: masked anyway
        c[bb] = cq * (g ? kb : ka);
      }
    } else {
      const float c0 = cq * kscale[min(2 * t, a.nbk - 1)];
      const float c1 = cq * kscale[min(2 * t + 1, a.nbk - 1)];   // past Nk: masked anyway
      c[0] = c[1] = c0;
      c[2] = c[3] = c1;
    }
    __builtin_amdgcn_s_setprio(0);
    softmax_phase<D, FP8, CAUSAL, decltype(masked)::value, FINE, T>(s, lane, t * kBkv, qi, nk, c, st.m, pt);
  };
#if SAGE_PHASE_TRACE
  // Diagnostic build only: per-wave shader-clock sums of the matrix phases,
  // the softmax phases and the two barriers' waits, the pair count and the
  // schedule's total; stored over the output at the end (see below).
  uint64_t tr[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint64_t tr_start = __builtin_readcyclecounter();
#if SAGE_PHASE_TRACE >= 2
  tr[6] = tr_start - tr_entry;                   // from kernel entry: work split, Q and first K tile loaded
#endif
  auto timed = [&](int slot, const auto& f) __attribute__((always_inline)) {
    const uint64_t t0 = __builtin_readcyclecounter();
    f();
    tr[slot] += __builtin_readcyclecounter() - t0;
  };
  auto x_tr = [&](auto par, int t, bool pv, bool qk) __attribute__((always_inline)) {
    timed(0, [&] { x_phase(par, t, pv, qk); });
  };
  auto xl_tr = [&](auto par, int t) __attribute__((always_inline)) { timed(0, [&] { x_phase_loading(par, t); }); };
  auto xr_tr = [&](int t, bool pv, bool qk) __attribute__((always_inline)) {
    timed(0, [&] { x_phase_rt(t, pv, qk); });
  };
  auto y_tr = [&](int t, auto masked) __attribute__((always_inline)) { timed(1, [&] { y_phase(t, masked); }); };
  auto ba_tr = [&]() __attribute__((always_inline)) { timed(2, [] { barrier_only(); }); };
  auto bw_tr = [&]() __attribute__((always_inline)) {
    timed(3, [] { wait_loads_barrier(); });
    tr[4] += 1;
  };
  run_pingpong(grp, n_g, n_wg, x_tr, xl_tr, xr_tr, y_tr, loads_k, loads_v, loads_k_rt, loads_v_rt, ba_tr, bw_tr);
  const uint64_t tr_sched_end = __builtin_readcyclecounter();
  tr[5] = tr_sched_end - tr_start;
#else
  run_pingpong(grp, n_g, n_wg, x_phase, x_phase_loading, x_phase_rt, y_phase, loads_k, loads_v, loads_k_rt,
               loads_v_rt);
#endif
  __builtin_amdgcn_s_setprio(0);

  // Epilogue: normalise, undo the V scale, round, store in the caller's layout.
  if (qi < nq) {
    // (the FP8 path's row sum is already complete in both lanes of a query; a
    //  sequence of a packed batch without keys gets zero rows)
    const float l = FP8 ? st.l : pair_sum(st.l);
    const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (int64_t)b * a.ogeo.batch_stride +
                     (int64_t)h * a.ogeo.head_stride + (o_tok + qi) * a.ogeo.tok_stride;
    const float* vs = FP8 ? a.v_scale + (int64_t)bhk * D : nullptr;
#pragma unroll
    for (int cb = 0; cb < NT; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = cb * 32 + 8 * j + 4 * g;
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = st.o[cb][4 * j + i] * inv_l;
        if (FP8 && l > 0.0f) {   // (a row without keys is exactly zero; its V scales may be unset)
          const f32x4 sv4 = *reinterpret_cast<const f32x4*>(vs + ch);
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] *= sv4[i];
        }
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2) w[i / 2] = (uint32_t)T::from_f32(x[i]) | ((uint32_t)T::from_f32(x[i + 1]) << 16);
        *reinterpret_cast<i32x2*>(orow + ch) = i32x2{(int)w[0], (int)w[1]};
      }
    }
  }
#if SAGE_PHASE_TRACE
  // Each wave's sums (low 32 bits) replace the output of the work-group's
  // first query row of this head (dense HND batches, d = 128): uint32 word
  // 8*wave + i. Level 2 adds slot 6 (cycles before the schedule), slot 7 (the
  // epilogue's issue time) and, from wave 0 in the second row, the
  // work-group's entry and exit times (the 100 MHz constant clock) and its
  // compute unit (XCC, shader engine, CU); its extra live values cost the
  // schedule some cycles per pair, so level 1 is the one for the phases.
#if SAGE_PHASE_TRACE >= 2
  tr[7] = __builtin_readcyclecounter() - tr_sched_end;
#else
  (void)tr_sched_end;
#endif
  __syncthreads();
  if constexpr (D == 128) {
    if (lane == 0 && !a.seq) {
      uint32_t* row = reinterpret_cast<uint32_t*>(a.o) + ((int64_t)bh * a.Nq + 2 * qp * kBq) * (D / 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) row[8 * wave + i] = (uint32_t)tr[i];
#if SAGE_PHASE_TRACE >= 2
      const uint64_t rt_exit = __builtin_amdgcn_s_memrealtime();
      if (wave == 0 && 2 * qp * kBq + 1 < a.Nq) {
        row += D / 2;
        row[0] = (uint32_t)rt_entry;
        row[1] = (uint32_t)(rt_entry >> 32);
        row[2] = (uint32_t)rt_exit;
        row[3] = (uint32_t)(rt_exit >> 32);
        row[4] = __smid();
      }
#endif
    }
  }
#endif
}

// Per-block Q/K scales.
template <int D, bool FP8, bool CAUSAL, typename T>
__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnArgs a) {
  attn_fwd_body<D, FP8, CAUSAL, T, false>(a);
}

// Per-thread Q/K scales: one per query and one per 16 keys.
template <int D, bool FP8, bool CAUSAL, typename T>
__global__ __launch_bounds__(512, 1) void attn_fwd_fine_kernel(AttnArgs a) {
  attn_fwd_body<D, FP8, CAUSAL, T, true>(a);
}

// INT32 S = Q8 K8^T through the same staging layout and matrix-core tile code.
template <int D>
__global__ __launch_bounds__(256) void debug_qk_kernel(DebugQKArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t s_k[kBkv * D];
  const int n_qt = (a.Nq + kBq - 1) / kBq;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int bhk = b * a.Hkv + h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5;
  const int qi = qt * kBq + wave * 32 + (lane & 31);
  i32x4 qreg[D / 32];
  load_q_operand<D>(a.q8 + (int64_t)bh * a.Nq * D, a.Nq, qi, g, qreg);
  const auto rk = make_rsrc(a.k8 + (int64_t)bhk * a.Nk * D, (uint32_t)a.Nk * D);
  for (int k0 = 0; k0 < a.Nk; k0 += kBkv) {
    __syncthreads();
    for (int ci = tid; ci < kBkv * D / 16; ci += 256)
      *reinterpret_cast<i32x4*>(s_k + k_lds_off<D>(ci / (D / 16), ci % (D / 16))) =
          buf_load16(rk, (uint32_t)(k0 + ci / (D / 16)) * D + (ci % (D / 16)) * 16);
    __syncthreads();
    i32x16 s[kBlocks];
    qk_tile<D>(s_k, qreg, lane, s, i32x16{});
    if (qi < a.Nq) {
      int32_t* row = a.s_out + ((int64_t)bh * a.Nq + qi) * a.Nk;
#pragma unroll
      for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * bb + 16 * g + r;
          if (key < a.Nk) row[key] = s[bb][r];
        }
    }
  }
}

// --------------------------------------------------------------- launchers
template <int D, bool FP8, bool CAUSAL, typename T>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  const int n_qp = (a.Nq + 2 * kBq - 1) / (2 * kBq);
  const int grid = a.seq ? a.n_owner * a.Hq : n_qp * a.B * a.Hq;   // packed: the work list per head
  if (a.fine)
    hipLaunchKernelGGL((attn_fwd_fine_kernel<D, FP8, CAUSAL, T>), dim3(grid), dim3(64 * kWaves), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, FP8, CAUSAL, T>), dim3(grid), dim3(64 * kWaves), 0, st, a);
  return hipGetLastError();
}

template <int D, bool FP8, typename T>
static hipError_t launch_attn_c(const AttnArgs& a, hipStream_t st) {
  return a.causal ? launch_attn_t<D, FP8, true, T>(a, st) : launch_attn_t<D, FP8, false, T>(a, st);
}

template <int D, typename T>
static hipError_t launch_attn_p(const AttnArgs& a, hipStream_t st) {
  return a.fp8 ? launch_attn_c<D, true, T>(a, st) : launch_attn_c<D, false, T>(a, st);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.Nq == 0) return hipSuccess;
  if (a.bf16) return a.D == 64 ? launch_attn_p<64, BF16>(a, st) : launch_attn_p<128, BF16>(a, st);
  return a.D == 64 ? launch_attn_p<64, F16>(a, st) : launch_attn_p<128, F16>(a, st);
}

hipError_t launch_debug_qk(const DebugQKArgs& a, hipStream_t st) {
  if (a.Nq == 0 || a.Nk == 0) return hipSuccess;
  const int grid = ((a.Nq + kBq - 1) / kBq) * a.B * a.Hq;
  if (a.D == 64)
    hipLaunchKernelGGL((debug_qk_kernel<64>), dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((debug_qk_kernel<128>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sage
