// Fused quantised attention forward for gfx950.
//
// One work-group = 4 waves = 128 queries of one (batch, query head); each wave
// owns 32 queries and walks the KV sequence in tiles of 64 keys, which all four
// waves share through LDS (double-buffered, one barrier per tile).
//
// Per wave and tile (SageAttention's hot loop: INT8 QK^T, online softmax, P in
// FP8 or FP16, PV with two-level accumulation -- thu-ml/SageAttention repo card,
// "How it works"; heatdrop.ai review, "The interesting bit"):
//   1. S^T[64 keys x 32 queries] = K8 . Q8^T on the INT8 matrix cores (INT32
//      accumulation). Computing the transpose puts one query per lane: lane l
//      holds query l % 32 and 16 keys per 32-key block, so every row reduction
//      is in-lane plus one exchange with lane l ^ 32.
//   2. Dequantise with c = s_q * s_k * sm_scale * log2(e) (one scalar per tile:
//      the tile is one K quantisation block, the work-group one Q block), mask
//      (causal diagonal / ragged tail), online softmax in the log2 domain.
//   3. P -> e4m3 (scaled by 448 through the exponent) or fp16/bf16, packed
//      straight from registers into the B operand of the PV product: the K rows
//      of step 1 are permuted so that each lane's keys are contiguous, exactly
//      the key order the PV operand needs.
//   4. R = V^T . P^T on the FP8 (or FP16/BF16) matrix cores into a fresh
//      accumulator (level 1), then O = alpha * O + R in fp32 (level 2).
// Epilogue: O * s_v[c] / l (FP8) or O / l, rounded to the input dtype and
// stored in the caller's layout.
#include <climits>
#include <type_traits>

#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kBq = 128;   // queries per work-group == the Q quantisation block

// --------------------------------------------------------------- LDS layouts
// K tile: [64 keys][D bytes]; 16-byte chunks XOR-swizzled per row so that the
// 8 rows read by 8 consecutive lanes land in 8 different bank groups.
__device__ __forceinline__ int key_swz(int row) { return (row & 3) | (((row >> 4) & 1) << 2); }
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int chunk) {
  return row * D + ((chunk ^ (key_swz(row) & (D / 16 - 1))) << 4);
}
// A row m of a 32-key block reads key key_perm(m); the S^T result then holds
// keys 16*g .. 16*g+15 of the block in lane group g, in element order.
__device__ __forceinline__ int key_perm(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }
// V^T tile: [D channels][64 keys] of 1 (e4m3) or 2 (fp16/bf16) bytes.
template <bool FP8>
__device__ __forceinline__ int v_lds_off(int row, int chunk) {
  if (FP8) return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4);
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ i32x4 lds16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }

// --------------------------------------------------------------- tile staging
template <int D, bool FP8>
struct TileStage {
  static constexpr int kChunks = 64 * D / 16;
  static constexpr int kPerThread = kChunks / 256;
  static constexpr int kVRowB = FP8 ? 64 : 128;
  static constexpr int kVChunks = D * kVRowB / 16;
  static constexpr int vPerThread = kVChunks / 256;
  i32x4 kr[kPerThread];
  i32x4 vr[vPerThread];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rk, const uint8_t* vbase, int n_pad, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int ci = i * 256 + tid;
      const int row = ci / (D / 16), chunk = ci % (D / 16);
      kr[i] = buf_load16(rk, (uint32_t)(k0 + row) * D + chunk * 16);   // rows >= Nk read as 0
    }
    constexpr int eb = FP8 ? 1 : 2;
#pragma unroll
    for (int i = 0; i < vPerThread; ++i) {
      const int ci = i * 256 + tid;
      const int row = ci / (kVRowB / 16), chunk = ci % (kVRowB / 16);
      vr[i] = *reinterpret_cast<const i32x4*>(vbase + ((int64_t)row * n_pad + k0) * eb + chunk * 16);
    }
  }
  __device__ __forceinline__ void store(int8_t* sk, uint8_t* sv, int tid) const {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int ci = i * 256 + tid;
      *reinterpret_cast<i32x4*>(sk + k_lds_off<D>(ci / (D / 16), ci % (D / 16))) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < vPerThread; ++i) {
      const int ci = i * 256 + tid;
      *reinterpret_cast<i32x4*>(sv + v_lds_off<FP8>(ci / (kVRowB / 16), ci % (kVRowB / 16))) = vr[i];
    }
  }
};

// S^T for keys [k0, k0+64) of the staged tile against this wave's queries.
template <int D>
__device__ __forceinline__ void qk_tile(const int8_t* sk, const i32x4* qreg, int lane, i32x16& s0, i32x16& s1) {
  const int g = lane >> 5, m = lane & 31;
  const int r0 = key_perm(m), r1 = 32 + key_perm(m);
  s0 = i32x16{};
  s1 = i32x16{};
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const i32x4 ka = lds16(sk + k_lds_off<D>(r0, 2 * t + g));
    const i32x4 kb = lds16(sk + k_lds_off<D>(r1, 2 * t + g));
    s0 = mfma_i8(ka, qreg[t], s0);
    s1 = mfma_i8(kb, qreg[t], s1);
  }
}

template <int D>
__device__ __forceinline__ void load_q_operand(const int8_t* q8_head, int nq, int qi, int g, i32x4* qreg) {
  const auto rq = make_rsrc(q8_head, (uint32_t)nq * D);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) qreg[t] = buf_load16(rq, (uint32_t)qi * D + 32 * t + 16 * g);
}

// --------------------------------------------------------------- the kernel
template <int D, bool FP8, bool CAUSAL, typename T>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int NT = D / 32;
  using Stage = TileStage<D, FP8>;
  __shared__ __attribute__((aligned(16))) int8_t s_k[2][64 * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][D * Stage::kVRowB];

  // Work decomposition. Work-groups are dealt round-robin to the 8 XCDs; give
  // each XCD a contiguous range of (head, q-tile) work so the work-groups that
  // share an XCD's L2 stream the same head's K/V tiles.
  const int n_qt = (a.Nq + kBq - 1) / kBq;
  const int total = n_qt * a.B * a.Hq;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  const int bh = id / n_qt;
  int qt = id % n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;            // longest rows first
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int bhk = b * a.Hkv + h / (a.Hq / a.Hkv);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int q0w = qt * kBq + wave * 32;
  const int qi = q0w + n;

  i32x4 qreg[NT];
  load_q_operand<D>(a.q8 + (int64_t)bh * a.Nq * D, a.Nq, qi, g, qreg);
  const float cq = a.q_scale[(int64_t)bh * a.nbq + qt] * a.scale_log2;
  const float* kscale = a.k_scale + (int64_t)bhk * a.nbk;

  const int kv_end = CAUSAL ? min(a.Nk, (qt + 1) * kBq) : a.Nk;
  const int n_kt = (kv_end + 63) / 64;
  // tiles this wave computes (waves entirely past Nq only help stage tiles)
  const int n_kt_wave = q0w >= a.Nq ? 0 : CAUSAL ? (min(a.Nk, q0w + 32) + 63) / 64 : n_kt;

  const auto rk = make_rsrc(a.k8 + (int64_t)bhk * a.Nk * D, (uint32_t)a.Nk * D);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vt) + (int64_t)bhk * D * a.n_pad * (FP8 ? 1 : 2);

  Stage stage;
  stage.load(rk, vbase, a.n_pad, 0, tid);
  stage.store(s_k[0], s_v[0], tid);
  __syncthreads();

  f32x16 o_acc[NT];
#pragma unroll
  for (int cb = 0; cb < NT; ++cb) o_acc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float bias_p = FP8 ? kLog2E4m3Max : 0.0f;   // P8 = e4m3(448 * P~) via the exponent

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) stage.load(rk, vbase, a.n_pad, (kt + 1) * 64, tid);
    if (kt < n_kt_wave) {
      const int k0 = kt * 64;
      i32x16 s0, s1;
      qk_tile<D>(s_k[buf], qreg, lane, s0, s1);

      const bool need_mask = (k0 + 64 > a.Nk) || (CAUSAL && k0 + 63 > q0w);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key0 = k0 + 16 * g + r, key1 = key0 + 32;
          if (key0 >= a.Nk || (CAUSAL && key0 > qi)) s0[r] = INT_MIN;
          if (key1 >= a.Nk || (CAUSAL && key1 > qi)) s1[r] = INT_MIN;
        }
      }
      int mx = INT_MIN;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = max(mx, max(s0[r], s1[r]));
      const float c = cq * kscale[kt];             // tile == one K quantisation block
      const float m_new = fmaxf(m_run, pair_max((float)mx * c));
      const float alpha = fast_exp2(m_run - m_new);
      const float bias = bias_p - m_new;

      float p0[16], p1[16];
      float lsum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p0[r] = fast_exp2(__builtin_fmaf((float)s0[r], c, bias));
        p1[r] = fast_exp2(__builtin_fmaf((float)s1[r], c, bias));
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (s0[r] == INT_MIN) p0[r] = 0.0f;
          if (s1[r] == INT_MIN) p1[r] = 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) lsum += p0[r] + p1[r];
      l_run = alpha * l_run + lsum;
      m_run = m_new;

      const uint8_t* sv = s_v[buf];
      if constexpr (FP8) {
        i32x8 pk;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0[4 * w], p0[4 * w + 1], 0, false);
          pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p0[4 * w + 2], p0[4 * w + 3], x, true);
          int y = __builtin_amdgcn_cvt_pk_fp8_f32(p1[4 * w], p1[4 * w + 1], 0, false);
          pk[4 + w] = __builtin_amdgcn_cvt_pk_fp8_f32(p1[4 * w + 2], p1[4 * w + 3], y, true);
        }
#pragma unroll
        for (int cb = 0; cb < NT; ++cb) {
          const int row = cb * 32 + n;
          const i32x4 lo = lds16(sv + v_lds_off<true>(row, g));
          const i32x4 hi = lds16(sv + v_lds_off<true>(row, 2 + g));
          const i32x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const f32x16 r = mfma_fp8(va, pk, f32x16{});            // level 1
#pragma unroll
          for (int e = 0; e < 16; ++e) o_acc[cb][e] = __builtin_fmaf(alpha, o_acc[cb][e], r[e]);  // level 2
        }
      } else {
        using H8 = typename std::conditional<std::is_same<T, BF16>::value, bf16x8, f16x8>::type;
        using HS = typename std::conditional<std::is_same<T, BF16>::value, __bf16, _Float16>::type;
        H8 ph[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ph[0][e] = (HS)p0[e];
          ph[1][e] = (HS)p0[8 + e];
          ph[2][e] = (HS)p1[e];
          ph[3][e] = (HS)p1[8 + e];
        }
#pragma unroll
        for (int cb = 0; cb < NT; ++cb) {
          const int row = cb * 32 + n;
          f32x16 r = f32x16{};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const i32x4 raw = lds16(sv + v_lds_off<false>(row, 2 * g + (u & 1) + 4 * (u >> 1)));
            r = mfma_half(__builtin_bit_cast(H8, raw), ph[u], r);   // level 1
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) o_acc[cb][e] = __builtin_fmaf(alpha, o_acc[cb][e], r[e]);  // level 2
        }
      }
    }
    if (kt + 1 < n_kt) stage.store(s_k[buf ^ 1], s_v[buf ^ 1], tid);
    __syncthreads();
  }

  // Epilogue: normalise, undo the V scale, round, store in the caller's layout.
  if (qi < a.Nq) {
    const float inv_l = 1.0f / pair_sum(l_run);
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + (int64_t)b * a.ogeo.batch_stride +
                     (int64_t)h * a.ogeo.head_stride + (int64_t)qi * a.ogeo.tok_stride;
    const float* vs = FP8 ? a.v_scale + (int64_t)bhk * D : nullptr;
#pragma unroll
    for (int cb = 0; cb < NT; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = cb * 32 + 8 * j + 4 * g;
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          float x0 = o_acc[cb][4 * j + i] * inv_l, x1 = o_acc[cb][4 * j + i + 1] * inv_l;
          if (FP8) {
            x0 *= vs[ch + i];
            x1 *= vs[ch + i + 1];
          }
          w[i / 2] = (uint32_t)T::from_f32(x0) | ((uint32_t)T::from_f32(x1) << 16);
        }
        *reinterpret_cast<i32x2*>(orow + ch) = i32x2{(int)w[0], (int)w[1]};
      }
    }
  }
}

// INT32 S = Q8 K8^T through the same staging and matrix-core tile code.
template <int D>
__global__ __launch_bounds__(256) void debug_qk_kernel(DebugQKArgs a) {
  __shared__ __attribute__((aligned(16))) int8_t s_k[64 * D];
  const int n_qt = (a.Nq + kBq - 1) / kBq;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int bhk = b * a.Hkv + h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int qi = qt * kBq + wave * 32 + n;
  i32x4 qreg[D / 32];
  load_q_operand<D>(a.q8 + (int64_t)bh * a.Nq * D, a.Nq, qi, g, qreg);
  const auto rk = make_rsrc(a.k8 + (int64_t)bhk * a.Nk * D, (uint32_t)a.Nk * D);
  for (int k0 = 0; k0 < a.Nk; k0 += 64) {
    __syncthreads();
    for (int ci = tid; ci < 64 * D / 16; ci += 256)
      *reinterpret_cast<i32x4*>(s_k + k_lds_off<D>(ci / (D / 16), ci % (D / 16))) =
          buf_load16(rk, (uint32_t)(k0 + ci / (D / 16)) * D + (ci % (D / 16)) * 16);
    __syncthreads();
    i32x16 s0, s1;
    qk_tile<D>(s_k, qreg, lane, s0, s1);
    if (qi < a.Nq) {
      int32_t* row = a.s_out + ((int64_t)bh * a.Nq + qi) * a.Nk;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key0 = k0 + 16 * g + r, key1 = key0 + 32;
        if (key0 < a.Nk) row[key0] = s0[r];
        if (key1 < a.Nk) row[key1] = s1[r];
      }
    }
  }
}

// --------------------------------------------------------------- launchers
template <int D, bool FP8, bool CAUSAL, typename T>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  const int n_qt = (a.Nq + kBq - 1) / kBq;
  const int grid = n_qt * a.B * a.Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<D, FP8, CAUSAL, T>), dim3(grid), dim3(256), 0, st, a);
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
