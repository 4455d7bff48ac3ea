// Internal (C++) interface between the C-ABI front end and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

// Element strides of a [B, H, N, d] tensor in either user layout
// (HND: token stride d; NHD: token stride H*d). The channel stride is 1.
struct TensorGeom {
  int64_t batch_stride;
  int64_t head_stride;
  int64_t tok_stride;
};

// One sequence of a packed variable-length batch (tokens of all sequences
// concatenated, [total, H, d]): its query and key token ranges and the first
// column of its keys in the padded V^T rows. Written by the plan kernel from
// the caller's cu_seqlens, clamped so that every range lies inside the packed
// tensors and the padded V^T rows.
struct SeqSpan {
  int32_t q0, nq, k0, nk, kp0;
  int32_t qp0;          // index of its first query pair (256 queries) in the packed work list
  int32_t reserved[2];
};

// Tokens per channel-statistics work-group: the K sums and V maxima are kept
// as one partial per (b, kv-head, chunk of kStatChunk tokens, channel), and
// the workspace is sized for them.
// (128 and 512 measured the same as 256 on one machine, within 0.5%.)
constexpr int kStatChunk = 256;

// The packed work list holds at most total_q / 256 + B query pairs.
inline int64_t varlen_qpair_bound(int64_t total_q, int64_t B) { return total_q / 256 + B; }

// Dense batches leave `seq` null. Packed batches set it, and then B is the
// sequence count, Nq/Nk the maximum sequence lengths (they size the grids and
// the per-sequence scale and partial strides), the geometries are the packed
// [total, H, d] ones, codes are stored [H][total][d] and V^T rows
// [Hkv][d][n_pad] with n_pad the padded-key bound.

struct QuantQKArgs {
  const void* q;
  const void* k;
  TensorGeom qgeo, kgeo;
  int B, Hq, Hkv, Nq, Nk, D;
  bool bf16;
  bool fine;           // per-thread scales (kFineBlkQ / kFineBlkK), else per block
  int8_t* q_codes;
  float* q_scale;
  int8_t* k_codes;
  float* k_scale;
  float* k_mean;
  double* ksum_part;   // [B*Hkv][ceil(Nk/256)][D]
  const SeqSpan* seq;  // packed batches only
  int total_q, total_k;
};

struct QuantVArgs {
  const void* v;
  TensorGeom vgeo;
  int B, Hkv, Nk, n_pad, D;
  bool bf16, fp8;
  void* out;           // FP8: e4m3 codes [B*Hkv][D][n_pad]; else 16-bit V^T [B*Hkv][D][n_pad]
  float* v_scale;      // FP8 only
  float* v_inv;        // FP8 only (448 / a_v)
  float* vmax_part;    // FP8 only: [B*Hkv][ceil(Nk/256)][D]
  const SeqSpan* seq;  // packed batches only
};

struct AttnArgs {
  const int8_t* q8;     // [B*Hq][Nq][D]
  const float* q_scale; // [B*Hq][nbq]
  const int8_t* k8;     // [B*Hkv][Nk][D]
  const float* k_scale; // [B*Hkv][nbk]
  const void* vt;       // [B*Hkv][D][n_pad]: e4m3 codes or 16-bit V^T
  const float* v_scale; // [B*Hkv][D] (FP8 only)
  void* o;
  TensorGeom ogeo;
  int B, Hq, Hkv, Nq, Nk, n_pad, D;
  int nbq, nbk;
  float scale_log2;     // sm_scale * log2(e)
  bool causal, bf16, fp8;
  bool fine;            // per-thread scales: q_scale per query, k_scale per 16 keys
  const SeqSpan* seq;   // packed batches only
  int total_q, total_k;
  const int32_t* qp_owner;  // packed batches: sequence of each work-list query pair, -1 past the end
  int n_owner;              // entries of qp_owner
};

struct DebugQKArgs {
  const int8_t* q8;
  const int8_t* k8;
  int32_t* s_out;       // [B*Hq][Nq][Nk]
  int B, Hq, Hkv, Nq, Nk, D;
};

// FP4 microscaling variant: MXFP4 codes two per byte, E8M0 scale bytes (the
// layouts are listed at the top of fp4_kernels.hip).
struct Fp4QuantArgs {
  const void* q;
  const void* k;
  const void* v;
  TensorGeom qgeo, kgeo, vgeo;
  int B, Hq, Hkv, Nq, Nk, n_pad, D;
  bool bf16;
  float q_mul;         // Q is quantised as fp32(q * q_mul): the score factor sm_scale * log2(e)
  uint8_t* q_codes;    // [B*Hq][Nq][D/2]
  uint8_t* q_scale;    // [B*Hq][Nq][D/32]
  uint8_t* k_codes;    // [B*Hkv][Nk][D/2]
  uint8_t* k_scale;    // [B*Hkv][Nk][D/32]
  float* k_mean;       // [B*Hkv][D]
  uint8_t* v_codes;    // [B*Hkv][D][n_pad/2]
  uint8_t* v_scale;    // [B*Hkv][n_pad/128][D][4]
  double* ksum_part;   // [B*Hkv][ceil(Nk/256)][D]
  const SeqSpan* seq;  // packed batches only: codes [H][total][.], k_mean [B][Hkv][D],
  int total_q, total_k;  // V^T [Hkv][D][n_pad/2] with each sequence's keys from column kp0
};

struct Fp4AttnArgs {
  const uint8_t* q4;
  const uint8_t* q_sc;
  const uint8_t* k4;
  const uint8_t* k_sc;
  const uint8_t* v4;
  const uint8_t* v_sc;
  void* o;
  TensorGeom ogeo;
  int B, Hq, Hkv, Nq, Nk, n_pad, D;   // (the score factor is already in the Q codes)
  bool causal, bf16;
  const SeqSpan* seq;                 // packed batches only (as for AttnArgs)
  int total_q, total_k;
  const int32_t* qp_owner;
  int n_owner;
};

hipError_t launch_varlen_plan(const int32_t* cu_q, const int32_t* cu_k, int B, int total_q, int total_k,
                              int max_q, int max_k, int n_pad, SeqSpan* out, int32_t* qp_owner, int n_owner,
                              hipStream_t st);
hipError_t launch_quant_qk(const QuantQKArgs& a, hipStream_t st);
hipError_t launch_quant_v(const QuantVArgs& a, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
hipError_t launch_debug_qk(const DebugQKArgs& a, hipStream_t st);
// K channel mean alone (the smoothing statistics of sage_quant_qk); packed
// batches pass their span table (B sequences, Nk the longest).
hipError_t launch_k_mean(const void* k, TensorGeom kgeo, int B, int Hkv, int Nk, int D, bool bf16, double* ksum_part,
                         float* k_mean, hipStream_t st, const SeqSpan* seq = nullptr);
hipError_t launch_quant_fp4(const Fp4QuantArgs& a, hipStream_t st);
hipError_t launch_attn_fp4(const Fp4AttnArgs& a, hipStream_t st);

}  // namespace sage
