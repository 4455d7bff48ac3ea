// C-ABI front end of libsage: argument validation, workspace layout, launches.
//
// Every entry point validates all arguments on the host before it makes any
// HIP call, so an invalid request enqueues nothing; this also lets the
// validation be exercised on a machine without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "sage.h"
#include "sage_device.h"
#include "sage_launch.h"

namespace {

using sage::TensorGeom;

using sage::kStatChunk;
constexpr int64_t kMaxSeq = int64_t(1) << 20;

struct Dims {
  int64_t B, Hq, Hkv, Nq, Nk, D;
  int64_t blk_q, blk_k;   // tokens per INT8 scale
  bool nhd, bf16, fine;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shape checks common to every entry point. `need_keys`: Nk must be > 0 when Nq > 0.
sage_status check_shape(const sage_shape* s, Dims* d) {
  if (!s) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->layout != SAGE_LAYOUT_HND && s->layout != SAGE_LAYOUT_NHD) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->dtype != SAGE_DTYPE_F16 && s->dtype != SAGE_DTYPE_BF16) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->qk_gran != SAGE_QK_PER_BLOCK && s->qk_gran != SAGE_QK_PER_THREAD) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->batch < 0 || s->heads_q < 1 || s->heads_kv < 1 || s->seq_q < 0 || s->seq_k < 0 || s->head_dim < 1)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (s->heads_q % s->heads_kv != 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->seq_q > kMaxSeq || s->seq_k > kMaxSeq) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->head_dim != 64 && s->head_dim != 128) return SAGE_ERR_UNSUPPORTED;
  d->B = s->batch;
  d->Hq = s->heads_q;
  d->Hkv = s->heads_kv;
  d->Nq = s->seq_q;
  d->Nk = s->seq_k;
  d->D = s->head_dim;
  d->nhd = s->layout == SAGE_LAYOUT_NHD;
  d->bf16 = s->dtype == SAGE_DTYPE_BF16;
  d->fine = s->qk_gran == SAGE_QK_PER_THREAD;
  d->blk_q = d->fine ? sage::kFineBlkQ : sage::kBlkQ;
  d->blk_k = d->fine ? sage::kFineBlkK : sage::kBlkK;
  // grid and buffer-offset limits: (b, head) pairs fit a grid dimension,
  // per-head slices fit a 32-bit byte offset
  if (d->B * d->Hq > (int64_t(1) << 24)) return SAGE_ERR_INVALID_ARGUMENT;
  return SAGE_OK;
}

TensorGeom geom(const Dims& d, int64_t H, int64_t N) {
  TensorGeom g;
  if (d.nhd) {
    g.batch_stride = N * H * d.D;
    g.head_stride = d.D;
    g.tok_stride = H * d.D;
  } else {
    g.batch_stride = H * N * d.D;
    g.head_stride = N * d.D;
    g.tok_stride = d.D;
  }
  return g;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  const uintptr_t xe = na > UINTPTR_MAX - x ? UINTPTR_MAX : x + na;   // (saturating ends)
  const uintptr_t ye = nb > UINTPTR_MAX - y ? UINTPTR_MAX : y + nb;
  return x < ye && y < xe;
}

// One buffer a call touches: base and byte count (a null base or zero count is
// skipped).
struct Span {
  const void* p;
  size_t n;
};

// True if two written buffers overlap, or a written buffer overlaps a read one.
bool aliased(std::initializer_list<Span> written, std::initializer_list<Span> read) {
  for (auto w = written.begin(); w != written.end(); ++w) {
    for (auto x = w + 1; x != written.end(); ++x)
      if (overlaps(w->p, w->n, x->p, x->n)) return true;
    for (const Span& r : read)
      if (overlaps(w->p, w->n, r.p, r.n)) return true;
  }
  return false;
}

// Workspace layout (each region 256-byte aligned), shared by all entry points.
struct Layout {
  size_t q_codes, q_scale, k_codes, k_scale, k_mean, vt, v_scale, v_inv, ksum, vmax, total;
};

Layout layout_for(const Dims& d, bool fp8) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t nbq = cdiv(d.Nq, d.blk_q), nbk = cdiv(d.Nk, d.blk_k);
  const int64_t npad = round_up(d.Nk, sage::kVPad);
  const int64_t chunks = cdiv(d.Nk, kStatChunk);
  L.q_codes = take(size_t(d.B * d.Hq * d.Nq * d.D));
  L.q_scale = take(size_t(d.B * d.Hq * nbq) * 4);
  L.k_codes = take(size_t(d.B * d.Hkv * d.Nk * d.D));
  L.k_scale = take(size_t(d.B * d.Hkv * nbk) * 4);
  L.k_mean = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.vt = take(size_t(d.B * d.Hkv * d.D * npad) * (fp8 ? 1 : 2));
  L.v_scale = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.v_inv = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.ksum = take(size_t(d.B * d.Hkv * chunks * d.D) * 8);
  L.vmax = take(size_t(d.B * d.Hkv * chunks * d.D) * 4);
  L.total = off;
  return L;
}

size_t qk_ws_bytes(const Dims& d) { return align256(size_t(d.B * d.Hkv * cdiv(d.Nk, kStatChunk) * d.D) * 8); }
size_t v_ws_bytes(const Dims& d) {
  return align256(size_t(d.B * d.Hkv * d.D) * 4) + align256(size_t(d.B * d.Hkv * cdiv(d.Nk, kStatChunk) * d.D) * 4);
}

// ---- packed variable-length batches
struct VDims {
  int64_t B, Hq, Hkv, D, total_q, total_k, max_q, max_k, n_pad;
  int64_t blk_q, blk_k;
  bool bf16, fine;
};

sage_status check_varlen_shape(const sage_varlen_shape* s, VDims* d) {
  if (!s) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->dtype != SAGE_DTYPE_F16 && s->dtype != SAGE_DTYPE_BF16) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->qk_gran != SAGE_QK_PER_BLOCK && s->qk_gran != SAGE_QK_PER_THREAD) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->batch < 0 || s->heads_q < 1 || s->heads_kv < 1 || s->head_dim < 1 || s->total_q < 0 || s->total_k < 0 ||
      s->max_seqlen_q < 0 || s->max_seqlen_k < 0)
    return SAGE_ERR_INVALID_ARGUMENT;
  if (s->heads_q % s->heads_kv != 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->max_seqlen_q > kMaxSeq || s->max_seqlen_k > kMaxSeq) return SAGE_ERR_INVALID_ARGUMENT;
  if (s->head_dim != 64 && s->head_dim != 128) return SAGE_ERR_UNSUPPORTED;
  d->B = s->batch;
  d->Hq = s->heads_q;
  d->Hkv = s->heads_kv;
  d->D = s->head_dim;
  d->total_q = s->total_q;
  d->total_k = s->total_k;
  d->max_q = s->max_seqlen_q;
  d->max_k = s->max_seqlen_k;
  d->bf16 = s->dtype == SAGE_DTYPE_BF16;
  d->fine = s->qk_gran == SAGE_QK_PER_THREAD;
  d->blk_q = d->fine ? sage::kFineBlkQ : sage::kBlkQ;
  d->blk_k = d->fine ? sage::kFineBlkK : sage::kBlkK;
  if (d->B * d->Hq > (int64_t(1) << 24)) return SAGE_ERR_INVALID_ARGUMENT;
  // padded V^T columns: every sequence's keys rounded up to the tile fit here
  if (d->total_k + (sage::kVPad - 1) * d->B > (int64_t(1) << 24) - sage::kVPad) return SAGE_ERR_INVALID_ARGUMENT;
  // attention grid: the query-pair work list for every query head
  if (sage::varlen_qpair_bound(d->total_q, d->B) * d->Hq > (int64_t(1) << 30)) return SAGE_ERR_INVALID_ARGUMENT;
  d->n_pad = round_up(d->total_k + (sage::kVPad - 1) * d->B, sage::kVPad);
  if (d->n_pad == 0) d->n_pad = sage::kVPad;
  return SAGE_OK;
}

// Workspace of a packed batch: the span table, codes [H][total][D], scales
// and partials with per-sequence strides from the maximum lengths, V^T rows
// [Hkv][D][n_pad].
struct VLayout {
  size_t spans, qp_owner, q_codes, q_scale, k_codes, k_scale, k_mean, vt, v_scale, v_inv, ksum, vmax, total;
};

VLayout varlen_layout_for(const VDims& d, bool fp8) {
  VLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t nbq = std::max<int64_t>(1, cdiv(d.max_q, d.blk_q)), nbk = std::max<int64_t>(1, cdiv(d.max_k, d.blk_k));
  const int64_t chunks = cdiv(d.max_k, kStatChunk);
  L.spans = take(size_t(d.B) * sizeof(sage::SeqSpan));
  L.qp_owner = take(size_t(sage::varlen_qpair_bound(d.total_q, d.B)) * 4);
  L.q_codes = take(size_t(d.Hq * d.total_q * d.D));
  L.q_scale = take(size_t(d.B * d.Hq * nbq) * 4);
  L.k_codes = take(size_t(d.Hkv * d.total_k * d.D));
  L.k_scale = take(size_t(d.B * d.Hkv * nbk) * 4);
  L.k_mean = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.vt = take(size_t(d.Hkv * d.D * d.n_pad) * (fp8 ? 1 : 2));
  L.v_scale = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.v_inv = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.ksum = take(size_t(d.B * d.Hkv * chunks * d.D) * 8);
  L.vmax = take(size_t(d.B * d.Hkv * chunks * d.D) * 4);
  L.total = off;
  return L;
}

// Packed [total, H, d] tensors: one long batch entry in NHD order.
TensorGeom packed_geom(int64_t H, int64_t D) {
  TensorGeom g;
  g.batch_stride = 0;
  g.head_stride = D;
  g.tok_stride = H * D;
  return g;
}

template <typename P>
P* at(void* base, size_t off) { return reinterpret_cast<P*>(static_cast<uint8_t*>(base) + off); }

sage_status from_hip(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

// Buffers of the quantisation stages of a packed batch.
struct VarlenBufs {
  sage::SeqSpan* spans;
  int32_t* qp_owner;
  int8_t* q_codes;
  float* q_scale;
  int8_t* k_codes;
  float* k_scale;
  float* k_mean;
  void* vt;
  float* v_scale;
  float* v_inv;
  double* ksum;
  float* vmax;
};

// Workspace of sage_quant_varlen: the span table and work list, 448/a_v, and
// the reduction partials (everything else goes to the caller's buffers).
struct VQLayout {
  size_t spans, qp_owner, v_inv, ksum, vmax, total;
};

VQLayout varlen_quant_layout_for(const VDims& d) {
  VQLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t chunks = cdiv(d.max_k, kStatChunk);
  L.spans = take(size_t(d.B) * sizeof(sage::SeqSpan));
  L.qp_owner = take(size_t(sage::varlen_qpair_bound(d.total_q, d.B)) * 4);
  L.v_inv = take(size_t(d.B * d.Hkv * d.D) * 4);
  L.ksum = take(size_t(d.B * d.Hkv * chunks * d.D) * 8);
  L.vmax = take(size_t(d.B * d.Hkv * chunks * d.D) * 4);
  L.total = off;
  return L;
}

// The plan kernel (span table from the device offsets) and the quantisation
// stages of a packed batch into `b`.
sage_status varlen_quant_launch(const VDims& d, bool fp8, const void* q, const void* k, const void* v,
                                const int32_t* cu_q, const int32_t* cu_k, const VarlenBufs& b, bool run_q,
                                bool run_kv, hipStream_t hs) {
  const int n_owner = int(sage::varlen_qpair_bound(d.total_q, d.B));
  hipError_t e = sage::launch_varlen_plan(cu_q, cu_k, int(d.B), int(d.total_q), int(d.total_k), int(d.max_q),
                                          int(d.max_k), int(d.n_pad), b.spans, b.qp_owner, n_owner, hs);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  sage::QuantQKArgs qa{};
  qa.q = q;
  qa.k = k;
  qa.qgeo = packed_geom(d.Hq, d.D);
  qa.kgeo = packed_geom(d.Hkv, d.D);
  qa.B = int(d.B), qa.Hq = int(d.Hq), qa.Hkv = int(d.Hkv), qa.Nq = int(d.max_q), qa.Nk = int(d.max_k);
  qa.D = int(d.D);
  qa.bf16 = d.bf16;
  qa.fine = d.fine;
  qa.q_codes = b.q_codes;
  qa.q_scale = b.q_scale;
  qa.k_codes = b.k_codes;
  qa.k_scale = b.k_scale;
  qa.k_mean = b.k_mean;
  qa.ksum_part = b.ksum;
  qa.seq = b.spans;
  qa.total_q = int(d.total_q);
  qa.total_k = int(d.total_k);
  if (!run_q) qa.Nq = 0;
  if (!run_kv) qa.Nk = 0;
  e = sage::launch_quant_qk(qa, hs);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  if (run_kv) {
    sage::QuantVArgs va{};
    va.v = v;
    va.vgeo = packed_geom(d.Hkv, d.D);
    va.B = int(d.B), va.Hkv = int(d.Hkv), va.Nk = int(d.max_k), va.D = int(d.D);
    va.n_pad = int(d.n_pad);
    va.bf16 = d.bf16;
    va.fp8 = fp8;
    va.out = b.vt;
    va.v_scale = b.v_scale;
    va.v_inv = b.v_inv;
    va.vmax_part = b.vmax;
    va.seq = b.spans;
    e = sage::launch_quant_v(va, hs);
    if (e != hipSuccess) return SAGE_ERR_HIP;
  }
  return SAGE_OK;
}

}  // namespace

// Workspace of sage_attn_fwd_noalloc: a fixed device array, one copy per GPU the
// library runs on, held until the process ends. Host code never uses its name
// as an address (on the host it is a stand-in symbol): the device address of
// each GPU's copy is taken once with hipGetSymbolAddress and kept below.
static __device__ __align__(256) uint8_t scratch[SAGE_NOALLOC_MAX_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call per device.
sage_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SAGE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SAGE_OK;
}

// The whole forward once the arguments are checked: statistics, quantisation,
// attention, all writing into `ws` (laid out by layout_for).
sage_status attn_fwd_launch(const Dims& d, const void* q, const void* k, const void* v, void* o, int32_t is_causal,
                            float sm_scale, bool fp8, void* workspace, hipStream_t hs) {
  const Layout L = layout_for(d, fp8);
  sage::QuantQKArgs qa{};
  qa.q = q;
  qa.k = k;
  qa.qgeo = geom(d, d.Hq, d.Nq);
  qa.kgeo = geom(d, d.Hkv, d.Nk);
  qa.B = int(d.B), qa.Hq = int(d.Hq), qa.Hkv = int(d.Hkv), qa.Nq = int(d.Nq), qa.Nk = int(d.Nk), qa.D = int(d.D);
  qa.bf16 = d.bf16;
  qa.fine = d.fine;
  qa.q_codes = at<int8_t>(workspace, L.q_codes);
  qa.q_scale = at<float>(workspace, L.q_scale);
  qa.k_codes = at<int8_t>(workspace, L.k_codes);
  qa.k_scale = at<float>(workspace, L.k_scale);
  qa.k_mean = at<float>(workspace, L.k_mean);
  qa.ksum_part = at<double>(workspace, L.ksum);
  hipError_t e = sage::launch_quant_qk(qa, hs);
  if (e != hipSuccess) return SAGE_ERR_HIP;

  sage::QuantVArgs va{};
  va.v = v;
  va.vgeo = geom(d, d.Hkv, d.Nk);
  va.B = int(d.B), va.Hkv = int(d.Hkv), va.Nk = int(d.Nk), va.D = int(d.D);
  va.n_pad = int(round_up(d.Nk, sage::kVPad));
  va.bf16 = d.bf16;
  va.fp8 = fp8;
  va.out = at<void>(workspace, L.vt);
  va.v_scale = at<float>(workspace, L.v_scale);
  va.v_inv = at<float>(workspace, L.v_inv);
  va.vmax_part = at<float>(workspace, L.vmax);
  e = sage::launch_quant_v(va, hs);
  if (e != hipSuccess) return SAGE_ERR_HIP;

  sage::AttnArgs aa{};
  aa.q8 = qa.q_codes;
  aa.q_scale = qa.q_scale;
  aa.k8 = qa.k_codes;
  aa.k_scale = qa.k_scale;
  aa.vt = va.out;
  aa.v_scale = va.v_scale;
  aa.o = o;
  aa.ogeo = geom(d, d.Hq, d.Nq);
  aa.B = int(d.B), aa.Hq = int(d.Hq), aa.Hkv = int(d.Hkv), aa.Nq = int(d.Nq), aa.Nk = int(d.Nk), aa.D = int(d.D);
  aa.n_pad = va.n_pad;
  aa.nbq = int(cdiv(d.Nq, d.blk_q));
  aa.nbk = int(cdiv(d.Nk, d.blk_k));
  aa.scale_log2 = sm_scale * sage::kLog2E;
  aa.causal = is_causal != 0;
  aa.bf16 = d.bf16;
  aa.fp8 = fp8;
  aa.fine = d.fine;
  return from_hip(sage::launch_attn(aa, hs));
}

// Argument checks of the whole forward that do not involve the workspace.
// SAGE_OK with *noop set means there is nothing to do.
sage_status attn_fwd_check(const sage_shape* s, const void* q, const void* k, const void* v, void* o,
                           int32_t is_causal, float sm_scale, int32_t pv_dtype, Dims* d, bool* noop) {
  *noop = false;
  sage_status st = check_shape(s, d);
  if (st != SAGE_OK) return st;
  if (pv_dtype != SAGE_PV_FP16 && pv_dtype != SAGE_PV_FP8_E4M3) return SAGE_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID_ARGUMENT;
  if (d->B == 0 || d->Nq == 0) {
    *noop = true;
    return SAGE_OK;
  }
  if (d->Nk == 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (is_causal && d->Nq != d->Nk) return SAGE_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return SAGE_ERR_INVALID_ARGUMENT;
  return SAGE_OK;
}

// ---- FP4 microscaling variant
// Byte counts of the MXFP4 buffers of shape `d` (layouts in include/sage.h).
struct Fp4Sizes {
  size_t q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, ksum;
};

Fp4Sizes fp4_sizes(const Dims& d) {
  const int64_t npad = round_up(d.Nk, sage::kVPad);
  Fp4Sizes z;
  z.q_codes = size_t(d.B * d.Hq * d.Nq * d.D / 2);
  z.q_scale = size_t(d.B * d.Hq * d.Nq * d.D / 32);
  z.k_codes = size_t(d.B * d.Hkv * d.Nk * d.D / 2);
  z.k_scale = size_t(d.B * d.Hkv * d.Nk * d.D / 32);
  z.k_mean = size_t(d.B * d.Hkv * d.D) * 4;
  z.v_codes = size_t(d.B * d.Hkv * d.D * npad / 2);
  z.v_scale = size_t(d.B * d.Hkv * d.D * npad / 32);
  z.ksum = size_t(d.B * d.Hkv * cdiv(d.Nk, kStatChunk) * d.D) * 8;
  return z;
}

struct Fp4Layout {
  size_t q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, ksum, total;
};

Fp4Layout fp4_layout_for(const Dims& d) {
  const Fp4Sizes z = fp4_sizes(d);
  Fp4Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.q_codes = take(z.q_codes);
  L.q_scale = take(z.q_scale);
  L.k_codes = take(z.k_codes);
  L.k_scale = take(z.k_scale);
  L.k_mean = take(z.k_mean);
  L.v_codes = take(z.v_codes);
  L.v_scale = take(z.v_scale);
  L.ksum = take(z.ksum);
  L.total = off;
  return L;
}

// Shape checks of the FP4 entry points: the MX blocks are fixed, so only the
// default granularity is accepted.
sage_status check_fp4_shape(const sage_shape* s, Dims* d) {
  sage_status st = check_shape(s, d);
  if (st != SAGE_OK) return st;
  if (d->fine) return SAGE_ERR_UNSUPPORTED;
  return SAGE_OK;
}

// The factor Q is scaled by before its quantisation: fp32(sm_scale * log2 e),
// the product taken in double and rounded once.
float fp4_score_factor(float sm_scale) { return (float)((double)sm_scale * 1.4426950408889634); }

sage::Fp4QuantArgs fp4_quant_args(const Dims& d, const void* q, const void* k, const void* v, float sm_scale,
                                  uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
                                  float* k_mean, uint8_t* v_codes, uint8_t* v_scale, double* ksum) {
  sage::Fp4QuantArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.qgeo = geom(d, d.Hq, d.Nq);
  a.kgeo = geom(d, d.Hkv, d.Nk);
  a.vgeo = geom(d, d.Hkv, d.Nk);
  a.B = int(d.B), a.Hq = int(d.Hq), a.Hkv = int(d.Hkv), a.Nq = int(d.Nq), a.Nk = int(d.Nk), a.D = int(d.D);
  a.n_pad = int(round_up(d.Nk, sage::kVPad));
  a.bf16 = d.bf16;
  a.q_mul = fp4_score_factor(sm_scale);
  a.q_codes = q_codes;
  a.q_scale = q_scale;
  a.k_codes = k_codes;
  a.k_scale = k_scale;
  a.k_mean = k_mean;
  a.v_codes = v_codes;
  a.v_scale = v_scale;
  a.ksum_part = ksum;
  return a;
}

sage::Fp4AttnArgs fp4_attn_args(const Dims& d, const uint8_t* q_codes, const uint8_t* q_scale,
                                const uint8_t* k_codes, const uint8_t* k_scale, const uint8_t* v_codes,
                                const uint8_t* v_scale, void* o, int32_t is_causal) {
  sage::Fp4AttnArgs a{};
  a.q4 = q_codes;
  a.q_sc = q_scale;
  a.k4 = k_codes;
  a.k_sc = k_scale;
  a.v4 = v_codes;
  a.v_sc = v_scale;
  a.o = o;
  a.ogeo = geom(d, d.Hq, d.Nq);
  a.B = int(d.B), a.Hq = int(d.Hq), a.Hkv = int(d.Hkv), a.Nq = int(d.Nq), a.Nk = int(d.Nk), a.D = int(d.D);
  a.n_pad = int(round_up(d.Nk, sage::kVPad));
  a.causal = is_causal != 0;
  a.bf16 = d.bf16;
  return a;
}

// FP4 variant of a packed batch: codes and scales [H][total][.], k_mean
// [sequence][Hkv][D], V^T codes [Hkv][D][n_pad/2] and scales
// [Hkv][n_pad/128][D][4] (each sequence from its span's column kp0).
struct Fp4VSizes {
  size_t q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, ksum, spans, qp_owner;
};

Fp4VSizes fp4_varlen_sizes(const VDims& d) {
  Fp4VSizes z;
  z.q_codes = size_t(d.Hq * d.total_q * d.D / 2);
  z.q_scale = size_t(d.Hq * d.total_q * d.D / 32);
  z.k_codes = size_t(d.Hkv * d.total_k * d.D / 2);
  z.k_scale = size_t(d.Hkv * d.total_k * d.D / 32);
  z.k_mean = size_t(d.B * d.Hkv * d.D) * 4;
  z.v_codes = size_t(d.Hkv * d.D * d.n_pad / 2);
  z.v_scale = size_t(d.Hkv * d.D * d.n_pad / 32);
  z.ksum = size_t(d.B * d.Hkv * cdiv(d.max_k, kStatChunk) * d.D) * 8;
  z.spans = size_t(d.B) * sizeof(sage::SeqSpan);
  z.qp_owner = size_t(sage::varlen_qpair_bound(d.total_q, d.B)) * 4;
  return z;
}

// Whole forward: every buffer in the workspace. Quantisation alone: the span
// table, the work list and the K sums (the codes go to the caller).
struct Fp4VLayout {
  size_t spans, qp_owner, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, ksum, total;
};

Fp4VLayout fp4_varlen_layout_for(const VDims& d, bool quant_only) {
  const Fp4VSizes z = fp4_varlen_sizes(d);
  Fp4VLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.spans = take(z.spans);
  L.qp_owner = take(z.qp_owner);
  L.ksum = take(z.ksum);
  if (!quant_only) {
    L.q_codes = take(z.q_codes);
    L.q_scale = take(z.q_scale);
    L.k_codes = take(z.k_codes);
    L.k_scale = take(z.k_scale);
    L.k_mean = take(z.k_mean);
    L.v_codes = take(z.v_codes);
    L.v_scale = take(z.v_scale);
  }
  L.total = off;
  return L;
}

sage_status check_fp4_varlen_shape(const sage_varlen_shape* s, VDims* d) {
  sage_status st = check_varlen_shape(s, d);
  if (st != SAGE_OK) return st;
  if (d->fine) return SAGE_ERR_UNSUPPORTED;
  return SAGE_OK;
}

// The plan kernel, then the MXFP4 stages of a packed batch.
sage_status fp4_varlen_quant_launch(const VDims& d, const void* q, const void* k, const void* v, const int32_t* cu_q,
                                    const int32_t* cu_k, float sm_scale, sage::SeqSpan* spans, int32_t* qp_owner,
                                    uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
                                    float* k_mean, uint8_t* v_codes, uint8_t* v_scale, double* ksum, bool run_q,
                                    bool run_kv, hipStream_t hs) {
  const int n_owner = int(sage::varlen_qpair_bound(d.total_q, d.B));
  hipError_t e = sage::launch_varlen_plan(cu_q, cu_k, int(d.B), int(d.total_q), int(d.total_k), int(d.max_q),
                                          int(d.max_k), int(d.n_pad), spans, qp_owner, n_owner, hs);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  sage::Fp4QuantArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.qgeo = packed_geom(d.Hq, d.D);
  a.kgeo = packed_geom(d.Hkv, d.D);
  a.vgeo = packed_geom(d.Hkv, d.D);
  a.B = int(d.B), a.Hq = int(d.Hq), a.Hkv = int(d.Hkv), a.Nq = int(d.max_q), a.Nk = int(d.max_k), a.D = int(d.D);
  a.n_pad = int(d.n_pad);
  a.bf16 = d.bf16;
  a.q_mul = fp4_score_factor(sm_scale);
  a.q_codes = q_codes;
  a.q_scale = q_scale;
  a.k_codes = k_codes;
  a.k_scale = k_scale;
  a.k_mean = k_mean;
  a.v_codes = v_codes;
  a.v_scale = v_scale;
  a.ksum_part = ksum;
  a.seq = spans;
  a.total_q = int(d.total_q);
  a.total_k = int(d.total_k);
  if (!run_q) a.Nq = 0;
  if (!run_kv) a.Nk = 0;
  return from_hip(sage::launch_quant_fp4(a, hs));
}

}  // namespace

extern "C" {

sage_status sage_block_sizes(int32_t head_dim, int32_t qk_gran, int32_t* blk_q, int32_t* blk_k, int32_t* bkv) {
  if (qk_gran != SAGE_QK_PER_BLOCK && qk_gran != SAGE_QK_PER_THREAD) return SAGE_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return SAGE_ERR_UNSUPPORTED;
  const bool fine = qk_gran == SAGE_QK_PER_THREAD;
  if (blk_q) *blk_q = fine ? sage::kFineBlkQ : sage::kBlkQ;
  if (blk_k) *blk_k = fine ? sage::kFineBlkK : sage::kBlkK;
  if (bkv) *bkv = sage::kBkv;
  return SAGE_OK;
}

int64_t sage_v_codes_stride(int32_t seq_k) { return seq_k <= 0 ? 0 : round_up(seq_k, sage::kVPad); }

size_t sage_quant_qk_workspace_bytes(const sage_shape* s) {
  Dims d;
  return check_shape(s, &d) == SAGE_OK ? qk_ws_bytes(d) : 0;
}

size_t sage_quant_v_workspace_bytes(const sage_shape* s) {
  Dims d;
  return check_shape(s, &d) == SAGE_OK ? v_ws_bytes(d) : 0;
}

size_t sage_workspace_bytes(const sage_shape* s, int32_t pv_dtype) {
  Dims d;
  if (check_shape(s, &d) != SAGE_OK) return 0;
  if (pv_dtype != SAGE_PV_FP16 && pv_dtype != SAGE_PV_FP8_E4M3) return 0;
  return layout_for(d, pv_dtype == SAGE_PV_FP8_E4M3).total;
}

sage_status sage_quant_qk(const sage_shape* s, const void* q, const void* k, int8_t* q_codes, float* q_scale,
                          int8_t* k_codes, float* k_scale, float* k_mean, void* workspace,
                          size_t workspace_bytes, void* stream) {
  Dims d;
  sage_status st = check_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (d.B == 0 || (d.Nq == 0 && d.Nk == 0)) return SAGE_OK;
  const bool has_q = d.Nq > 0, has_k = d.Nk > 0;
  if (has_q && (!q || !q_codes || !q_scale)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!k || !k_codes || !k_scale || !k_mean)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_q && (!aligned(q, 16) || !aligned(q_codes, 16) || !aligned(q_scale, 4))) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!aligned(k, 16) || !aligned(k_codes, 16) || !aligned(k_scale, 4) || !aligned(k_mean, 4)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k) {
    if (!workspace || !aligned(workspace, 256)) return SAGE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < qk_ws_bytes(d)) return SAGE_ERR_WORKSPACE;
  }
  {
    const size_t nq = has_q ? size_t(d.B * d.Hq * d.Nq * d.D) : 0, nk = has_k ? size_t(d.B * d.Hkv * d.Nk * d.D) : 0;
    const size_t sq = has_q ? size_t(d.B * d.Hq * cdiv(d.Nq, d.blk_q)) * 4 : 0;
    const size_t sk = has_k ? size_t(d.B * d.Hkv * cdiv(d.Nk, d.blk_k)) * 4 : 0;
    const size_t mk = has_k ? size_t(d.B * d.Hkv * d.D) * 4 : 0, wk = has_k ? qk_ws_bytes(d) : 0;
    if (aliased({{q_codes, nq}, {q_scale, sq}, {k_codes, nk}, {k_scale, sk}, {k_mean, mk}, {workspace, wk}},
                {{q, nq * 2}, {k, nk * 2}}))
      return SAGE_ERR_INVALID_ARGUMENT;
  }
  sage::QuantQKArgs a{};
  a.q = q;
  a.k = k;
  a.qgeo = geom(d, d.Hq, d.Nq);
  a.kgeo = geom(d, d.Hkv, d.Nk);
  a.B = int(d.B), a.Hq = int(d.Hq), a.Hkv = int(d.Hkv), a.Nq = int(d.Nq), a.Nk = int(d.Nk), a.D = int(d.D);
  a.bf16 = d.bf16;
  a.fine = d.fine;
  a.q_codes = q_codes;
  a.q_scale = q_scale;
  a.k_codes = k_codes;
  a.k_scale = k_scale;
  a.k_mean = k_mean;
  a.ksum_part = static_cast<double*>(workspace);
  return from_hip(sage::launch_quant_qk(a, static_cast<hipStream_t>(stream)));
}

sage_status sage_quant_v(const sage_shape* s, const void* v, uint8_t* v_codes, float* v_scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Dims d;
  sage_status st = check_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (d.B == 0 || d.Nk == 0) return SAGE_OK;
  if (!v || !v_codes || !v_scale || !workspace) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(v, 16) || !aligned(v_codes, 16) || !aligned(v_scale, 4) || !aligned(workspace, 256))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < v_ws_bytes(d)) return SAGE_ERR_WORKSPACE;
  if (aliased({{v_codes, size_t(d.B * d.Hkv * d.D * round_up(d.Nk, sage::kVPad))},
               {v_scale, size_t(d.B * d.Hkv * d.D) * 4}, {workspace, v_ws_bytes(d)}},
              {{v, size_t(d.B * d.Hkv * d.Nk * d.D) * 2}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  sage::QuantVArgs a{};
  a.v = v;
  a.vgeo = geom(d, d.Hkv, d.Nk);
  a.B = int(d.B), a.Hkv = int(d.Hkv), a.Nk = int(d.Nk), a.D = int(d.D);
  a.n_pad = int(round_up(d.Nk, sage::kVPad));
  a.bf16 = d.bf16;
  a.fp8 = true;
  a.out = v_codes;
  a.v_scale = v_scale;
  a.v_inv = static_cast<float*>(workspace);
  a.vmax_part = at<float>(workspace, align256(size_t(d.B * d.Hkv * d.D) * 4));
  return from_hip(sage::launch_quant_v(a, static_cast<hipStream_t>(stream)));
}

sage_status sage_attn_fwd(const sage_shape* s, const void* q, const void* k, const void* v, void* o,
                          int32_t is_causal, float sm_scale, int32_t pv_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  Dims d;
  bool noop = false;
  sage_status st = attn_fwd_check(s, q, k, v, o, is_causal, sm_scale, pv_dtype, &d, &noop);
  if (st != SAGE_OK || noop) return st;
  if (!workspace || !aligned(workspace, 256)) return SAGE_ERR_INVALID_ARGUMENT;
  const bool fp8 = pv_dtype == SAGE_PV_FP8_E4M3;
  const Layout L = layout_for(d, fp8);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  const size_t qbytes = size_t(d.B * d.Hq * d.Nq * d.D) * 2, kvbytes = size_t(d.B * d.Hkv * d.Nk * d.D) * 2;
  if (aliased({{o, qbytes}, {workspace, L.total}}, {{q, qbytes}, {k, kvbytes}, {v, kvbytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  return attn_fwd_launch(d, q, k, v, o, is_causal, sm_scale, fp8, workspace, static_cast<hipStream_t>(stream));
}

sage_status sage_attn_fwd_noalloc(const sage_shape* s, const void* q, const void* k, const void* v, void* o,
                                  int32_t is_causal, float sm_scale, int32_t pv_dtype, void* stream) {
  Dims d;
  bool noop = false;
  sage_status st = attn_fwd_check(s, q, k, v, o, is_causal, sm_scale, pv_dtype, &d, &noop);
  if (st != SAGE_OK || noop) return st;
  const bool fp8 = pv_dtype == SAGE_PV_FP8_E4M3;
  const Layout L = layout_for(d, fp8);
  if (L.total > size_t(SAGE_NOALLOC_MAX_WORKSPACE_BYTES)) return SAGE_ERR_WORKSPACE;
  const size_t qbytes = size_t(d.B * d.Hq * d.Nq * d.D) * 2, kvbytes = size_t(d.B * d.Hkv * d.Nk * d.D) * 2;
  if (aliased({{o, qbytes}}, {{q, qbytes}, {k, kvbytes}, {v, kvbytes}})) return SAGE_ERR_INVALID_ARGUMENT;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != SAGE_OK) return st;
  if (aliased({{o, qbytes}, {ws, L.total}}, {{q, qbytes}, {k, kvbytes}, {v, kvbytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  // Every workspace region is written by this call's kernels before any kernel
  // reads it (codes, scales, K mean, V^T with its zero padding, the reduction
  // partials), so the array's contents from an earlier call never leak in and
  // nothing needs clearing.
  return attn_fwd_launch(d, q, k, v, o, is_causal, sm_scale, fp8, ws, static_cast<hipStream_t>(stream));
}

size_t sage_varlen_workspace_bytes(const sage_varlen_shape* s, int32_t pv_dtype) {
  VDims d;
  if (check_varlen_shape(s, &d) != SAGE_OK) return 0;
  if (pv_dtype != SAGE_PV_FP16 && pv_dtype != SAGE_PV_FP8_E4M3) return 0;
  return varlen_layout_for(d, pv_dtype == SAGE_PV_FP8_E4M3).total;
}

sage_status sage_attn_fwd_varlen(const sage_varlen_shape* s, const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                                 int32_t is_causal, float sm_scale, int32_t pv_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  VDims d;
  sage_status st = check_varlen_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (pv_dtype != SAGE_PV_FP16 && pv_dtype != SAGE_PV_FP8_E4M3) return SAGE_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0 || d.total_q == 0 || d.max_q == 0) return SAGE_OK;
  const bool has_k = d.total_k > 0 && d.max_k > 0;   // (else every output row is zero; k, v may be NULL)
  if (!q || !o || !cu_seqlens_q || !cu_seqlens_k || !workspace || (has_k && (!k || !v)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(cu_seqlens_q, 4) ||
      !aligned(cu_seqlens_k, 4) || !aligned(workspace, 256))
    return SAGE_ERR_INVALID_ARGUMENT;
  const bool fp8 = pv_dtype == SAGE_PV_FP8_E4M3;
  const VLayout L = varlen_layout_for(d, fp8);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  const size_t qbytes = size_t(d.total_q * d.Hq * d.D) * 2, kvbytes = size_t(d.total_k * d.Hkv * d.D) * 2;
  const size_t cubytes = size_t(d.B + 1) * 4;
  if (aliased({{o, qbytes}, {workspace, L.total}},
              {{q, qbytes}, {k, kvbytes}, {v, kvbytes}, {cu_seqlens_q, cubytes}, {cu_seqlens_k, cubytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  VarlenBufs bufs{};
  bufs.spans = at<sage::SeqSpan>(workspace, L.spans);
  bufs.qp_owner = at<int32_t>(workspace, L.qp_owner);
  bufs.q_codes = at<int8_t>(workspace, L.q_codes);
  bufs.q_scale = at<float>(workspace, L.q_scale);
  bufs.k_codes = at<int8_t>(workspace, L.k_codes);
  bufs.k_scale = at<float>(workspace, L.k_scale);
  bufs.k_mean = at<float>(workspace, L.k_mean);
  bufs.vt = at<void>(workspace, L.vt);
  bufs.v_scale = at<float>(workspace, L.v_scale);
  bufs.v_inv = at<float>(workspace, L.v_inv);
  bufs.ksum = at<double>(workspace, L.ksum);
  bufs.vmax = at<float>(workspace, L.vmax);
  st = varlen_quant_launch(d, fp8, q, k, v, cu_seqlens_q, cu_seqlens_k, bufs, true, has_k, hs);
  if (st != SAGE_OK) return st;

  sage::AttnArgs aa{};
  aa.q8 = bufs.q_codes;
  aa.q_scale = bufs.q_scale;
  aa.k8 = bufs.k_codes;
  aa.k_scale = bufs.k_scale;
  aa.vt = bufs.vt;
  aa.v_scale = bufs.v_scale;
  aa.o = o;
  aa.ogeo = packed_geom(d.Hq, d.D);
  aa.B = int(d.B), aa.Hq = int(d.Hq), aa.Hkv = int(d.Hkv), aa.Nq = int(d.max_q), aa.Nk = int(d.max_k);
  aa.D = int(d.D);
  aa.n_pad = int(d.n_pad);
  aa.nbq = int(std::max<int64_t>(1, cdiv(d.max_q, d.blk_q)));
  aa.nbk = int(std::max<int64_t>(1, cdiv(d.max_k, d.blk_k)));
  aa.scale_log2 = sm_scale * sage::kLog2E;
  aa.causal = is_causal != 0;
  aa.bf16 = d.bf16;
  aa.fp8 = fp8;
  aa.fine = d.fine;
  aa.seq = bufs.spans;
  aa.total_q = int(d.total_q);
  aa.total_k = int(d.total_k);
  aa.qp_owner = bufs.qp_owner;
  aa.n_owner = int(sage::varlen_qpair_bound(d.total_q, d.B));
  return from_hip(sage::launch_attn(aa, hs));
}

size_t sage_quant_varlen_workspace_bytes(const sage_varlen_shape* s) {
  VDims d;
  if (check_varlen_shape(s, &d) != SAGE_OK) return 0;
  return varlen_quant_layout_for(d).total;
}

sage_status sage_quant_varlen(const sage_varlen_shape* s, int32_t pv_dtype, const void* q, const void* k,
                              const void* v, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale, float* k_mean,
                              void* v_prepared, float* v_scale, void* workspace, size_t workspace_bytes,
                              void* stream) {
  VDims d;
  sage_status st = check_varlen_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (pv_dtype != SAGE_PV_FP16 && pv_dtype != SAGE_PV_FP8_E4M3) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0) return SAGE_OK;
  const bool fp8 = pv_dtype == SAGE_PV_FP8_E4M3;
  const bool has_q = d.total_q > 0 && d.max_q > 0, has_k = d.total_k > 0 && d.max_k > 0;
  if (!cu_seqlens_q || !cu_seqlens_k || !workspace) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_q && (!q || !q_codes || !q_scale)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!k || !v || !k_codes || !k_scale || !k_mean || !v_prepared || (fp8 && !v_scale)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(workspace, 256)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_q && (!aligned(q, 16) || !aligned(q_codes, 16) || !aligned(q_scale, 4))) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, 16) || !aligned(k_scale, 4) ||
                !aligned(k_mean, 4) || !aligned(v_prepared, 16) || (fp8 && !aligned(v_scale, 4))))
    return SAGE_ERR_INVALID_ARGUMENT;
  const VQLayout L = varlen_quant_layout_for(d);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  const int64_t nbq = std::max<int64_t>(1, cdiv(d.max_q, d.blk_q)), nbk = std::max<int64_t>(1, cdiv(d.max_k, d.blk_k));
  const size_t nq = has_q ? size_t(d.Hq * d.total_q * d.D) : 0, nk = has_k ? size_t(d.Hkv * d.total_k * d.D) : 0;
  const size_t cubytes = size_t(d.B + 1) * 4;
  if (aliased({{q_codes, nq}, {q_scale, has_q ? size_t(d.B * d.Hq * nbq) * 4 : 0}, {k_codes, nk},
               {k_scale, has_k ? size_t(d.B * d.Hkv * nbk) * 4 : 0}, {k_mean, has_k ? size_t(d.B * d.Hkv * d.D) * 4 : 0},
               {v_prepared, has_k ? size_t(d.Hkv * d.D * d.n_pad) * (fp8 ? 1 : 2) : 0},
               {fp8 ? v_scale : nullptr, has_k ? size_t(d.B * d.Hkv * d.D) * 4 : 0}, {workspace, L.total}},
              {{q, nq * 2}, {k, nk * 2}, {v, nk * 2}, {cu_seqlens_q, cubytes}, {cu_seqlens_k, cubytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  VarlenBufs bufs{};
  bufs.spans = at<sage::SeqSpan>(workspace, L.spans);
  bufs.qp_owner = at<int32_t>(workspace, L.qp_owner);
  bufs.q_codes = q_codes;
  bufs.q_scale = q_scale;
  bufs.k_codes = k_codes;
  bufs.k_scale = k_scale;
  bufs.k_mean = k_mean;
  bufs.vt = v_prepared;
  bufs.v_scale = v_scale;
  bufs.v_inv = at<float>(workspace, L.v_inv);
  bufs.ksum = at<double>(workspace, L.ksum);
  bufs.vmax = at<float>(workspace, L.vmax);
  return varlen_quant_launch(d, fp8, q, k, v, cu_seqlens_q, cu_seqlens_k, bufs, has_q, has_k,
                             static_cast<hipStream_t>(stream));
}

sage_status sage_transpose_v(const sage_shape* s, const void* v, void* v_t, void* stream) {
  Dims d;
  sage_status st = check_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (d.B == 0 || d.Nk == 0) return SAGE_OK;
  if (!v || !v_t || !aligned(v, 16) || !aligned(v_t, 16)) return SAGE_ERR_INVALID_ARGUMENT;
  if (aliased({{v_t, size_t(d.B * d.Hkv * d.D * round_up(d.Nk, sage::kVPad)) * 2}},
              {{v, size_t(d.B * d.Hkv * d.Nk * d.D) * 2}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  sage::QuantVArgs a{};
  a.v = v;
  a.vgeo = geom(d, d.Hkv, d.Nk);
  a.B = int(d.B), a.Hkv = int(d.Hkv), a.Nk = int(d.Nk), a.D = int(d.D);
  a.n_pad = int(round_up(d.Nk, sage::kVPad));
  a.bf16 = d.bf16;
  a.fp8 = false;
  a.out = v_t;
  return from_hip(sage::launch_quant_v(a, static_cast<hipStream_t>(stream)));
}

sage_status sage_attn_fwd_codes(const sage_shape* s, const int8_t* q_codes, const float* q_scale,
                                const int8_t* k_codes, const float* k_scale, const void* v_prepared,
                                const float* v_scale, void* o, int32_t is_causal, float sm_scale,
                                int32_t pv_dtype, void* stream) {
  Dims d;
  sage_status st = check_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (pv_dtype != SAGE_PV_FP16 && pv_dtype != SAGE_PV_FP8_E4M3) return SAGE_ERR_INVALID_ARGUMENT;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0 || d.Nq == 0) return SAGE_OK;
  if (d.Nk == 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (is_causal && d.Nq != d.Nk) return SAGE_ERR_UNSUPPORTED;
  const bool fp8 = pv_dtype == SAGE_PV_FP8_E4M3;
  if (!q_codes || !q_scale || !k_codes || !k_scale || !v_prepared || !o || (fp8 && !v_scale))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_prepared, 16) || !aligned(o, 16) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || (fp8 && !aligned(v_scale, 16)))
    return SAGE_ERR_INVALID_ARGUMENT;
  const size_t obytes = size_t(d.B * d.Hq * d.Nq * d.D) * 2;
  const int64_t npad = round_up(d.Nk, sage::kVPad);
  if (aliased({{o, obytes}},
              {{q_codes, size_t(d.B * d.Hq * d.Nq * d.D)}, {q_scale, size_t(d.B * d.Hq * cdiv(d.Nq, d.blk_q)) * 4},
               {k_codes, size_t(d.B * d.Hkv * d.Nk * d.D)}, {k_scale, size_t(d.B * d.Hkv * cdiv(d.Nk, d.blk_k)) * 4},
               {v_prepared, size_t(d.B * d.Hkv * d.D * npad) * (fp8 ? 1 : 2)},
               {fp8 ? v_scale : nullptr, size_t(d.B * d.Hkv * d.D) * 4}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  sage::AttnArgs aa{};
  aa.q8 = q_codes;
  aa.q_scale = q_scale;
  aa.k8 = k_codes;
  aa.k_scale = k_scale;
  aa.vt = v_prepared;
  aa.v_scale = v_scale;
  aa.o = o;
  aa.ogeo = geom(d, d.Hq, d.Nq);
  aa.B = int(d.B), aa.Hq = int(d.Hq), aa.Hkv = int(d.Hkv), aa.Nq = int(d.Nq), aa.Nk = int(d.Nk), aa.D = int(d.D);
  aa.n_pad = int(npad);
  aa.nbq = int(cdiv(d.Nq, d.blk_q));
  aa.nbk = int(cdiv(d.Nk, d.blk_k));
  aa.scale_log2 = sm_scale * sage::kLog2E;
  aa.causal = is_causal != 0;
  aa.bf16 = d.bf16;
  aa.fp8 = fp8;
  aa.fine = d.fine;
  return from_hip(sage::launch_attn(aa, static_cast<hipStream_t>(stream)));
}

size_t sage_quant_fp4_workspace_bytes(const sage_shape* s) {
  Dims d;
  return check_fp4_shape(s, &d) == SAGE_OK ? qk_ws_bytes(d) : 0;
}

size_t sage_fp4_workspace_bytes(const sage_shape* s) {
  Dims d;
  return check_fp4_shape(s, &d) == SAGE_OK ? fp4_layout_for(d).total : 0;
}

sage_status sage_quant_fp4(const sage_shape* s, const void* q, const void* k, const void* v, float sm_scale,
                           uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale, float* k_mean,
                           uint8_t* v_codes, uint8_t* v_scale, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Dims d;
  sage_status st = check_fp4_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0 || (d.Nq == 0 && d.Nk == 0)) return SAGE_OK;
  const bool has_q = d.Nq > 0, has_k = d.Nk > 0;
  if (has_q && (!q || !q_codes || !q_scale)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!k || !v || !k_codes || !k_scale || !k_mean || !v_codes || !v_scale || !workspace))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (has_q && (!aligned(q, 16) || !aligned(q_codes, 16) || !aligned(q_scale, 4))) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, 16) || !aligned(k_scale, 4) ||
                !aligned(k_mean, 4) || !aligned(v_codes, 16) || !aligned(v_scale, 16) || !aligned(workspace, 256)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && workspace_bytes < qk_ws_bytes(d)) return SAGE_ERR_WORKSPACE;
  const Fp4Sizes z = fp4_sizes(d);
  const size_t qin = has_q ? size_t(d.B * d.Hq * d.Nq * d.D) * 2 : 0, kin = has_k ? size_t(d.B * d.Hkv * d.Nk * d.D) * 2 : 0;
  if (aliased({{q_codes, has_q ? z.q_codes : 0}, {q_scale, has_q ? z.q_scale : 0}, {k_codes, has_k ? z.k_codes : 0},
               {k_scale, has_k ? z.k_scale : 0}, {k_mean, has_k ? z.k_mean : 0}, {v_codes, has_k ? z.v_codes : 0},
               {v_scale, has_k ? z.v_scale : 0}, {workspace, has_k ? qk_ws_bytes(d) : 0}},
              {{q, qin}, {k, kin}, {v, kin}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  sage::Fp4QuantArgs a = fp4_quant_args(d, q, k, v, sm_scale, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes,
                                        v_scale, static_cast<double*>(workspace));
  if (!has_q) a.Nq = 0;
  if (!has_k) a.Nk = 0, a.n_pad = 0;
  return from_hip(sage::launch_quant_fp4(a, static_cast<hipStream_t>(stream)));
}

sage_status sage_attn_fwd_fp4_codes(const sage_shape* s, const uint8_t* q_codes, const uint8_t* q_scale,
                                    const uint8_t* k_codes, const uint8_t* k_scale, const uint8_t* v_codes,
                                    const uint8_t* v_scale, void* o, int32_t is_causal, void* stream) {
  Dims d;
  sage_status st = check_fp4_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0 || d.Nq == 0) return SAGE_OK;
  if (d.Nk == 0) return SAGE_ERR_INVALID_ARGUMENT;
  if (is_causal && d.Nq != d.Nk) return SAGE_ERR_UNSUPPORTED;
  if (!q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale || !o) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(o, 16) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 16))
    return SAGE_ERR_INVALID_ARGUMENT;
  const Fp4Sizes z = fp4_sizes(d);
  if (aliased({{o, size_t(d.B * d.Hq * d.Nq * d.D) * 2}},
              {{q_codes, z.q_codes}, {q_scale, z.q_scale}, {k_codes, z.k_codes}, {k_scale, (z.k_scale + 3) & ~size_t(3)},
               {v_codes, z.v_codes}, {v_scale, z.v_scale}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  return from_hip(sage::launch_attn_fp4(
      fp4_attn_args(d, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, o, is_causal),
      static_cast<hipStream_t>(stream)));
}

sage_status sage_attn_fwd_fp4(const sage_shape* s, const void* q, const void* k, const void* v, void* o,
                              int32_t is_causal, float sm_scale, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Dims d;
  bool noop = false;
  sage_status st = check_fp4_shape(s, &d);
  if (st != SAGE_OK) return st;
  st = attn_fwd_check(s, q, k, v, o, is_causal, sm_scale, SAGE_PV_FP16, &d, &noop);
  if (st != SAGE_OK || noop) return st;
  if (!workspace || !aligned(workspace, 256)) return SAGE_ERR_INVALID_ARGUMENT;
  const Fp4Layout L = fp4_layout_for(d);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  const size_t qbytes = size_t(d.B * d.Hq * d.Nq * d.D) * 2, kvbytes = size_t(d.B * d.Hkv * d.Nk * d.D) * 2;
  if (aliased({{o, qbytes}, {workspace, L.total}}, {{q, qbytes}, {k, kvbytes}, {v, kvbytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const sage::Fp4QuantArgs qa =
      fp4_quant_args(d, q, k, v, sm_scale, at<uint8_t>(workspace, L.q_codes), at<uint8_t>(workspace, L.q_scale),
                     at<uint8_t>(workspace, L.k_codes), at<uint8_t>(workspace, L.k_scale),
                     at<float>(workspace, L.k_mean), at<uint8_t>(workspace, L.v_codes),
                     at<uint8_t>(workspace, L.v_scale), at<double>(workspace, L.ksum));
  if (sage::launch_quant_fp4(qa, hs) != hipSuccess) return SAGE_ERR_HIP;
  return from_hip(sage::launch_attn_fp4(fp4_attn_args(d, qa.q_codes, qa.q_scale, qa.k_codes, qa.k_scale,
                                                      qa.v_codes, qa.v_scale, o, is_causal),
                                        hs));
}

size_t sage_fp4_varlen_workspace_bytes(const sage_varlen_shape* s) {
  VDims d;
  return check_fp4_varlen_shape(s, &d) == SAGE_OK ? fp4_varlen_layout_for(d, false).total : 0;
}

sage_status sage_attn_fwd_fp4_varlen(const sage_varlen_shape* s, const void* q, const void* k, const void* v,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o,
                                     int32_t is_causal, float sm_scale, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  VDims d;
  sage_status st = check_fp4_varlen_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0 || d.total_q == 0 || d.max_q == 0) return SAGE_OK;
  const bool has_k = d.total_k > 0 && d.max_k > 0;   // (else every output row is zero; k, v may be NULL)
  if (!q || !o || !cu_seqlens_q || !cu_seqlens_k || !workspace || (has_k && (!k || !v)))
    return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(cu_seqlens_q, 4) ||
      !aligned(cu_seqlens_k, 4) || !aligned(workspace, 256))
    return SAGE_ERR_INVALID_ARGUMENT;
  const Fp4VLayout L = fp4_varlen_layout_for(d, false);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  const size_t qbytes = size_t(d.total_q * d.Hq * d.D) * 2, kvbytes = size_t(d.total_k * d.Hkv * d.D) * 2;
  const size_t cubytes = size_t(d.B + 1) * 4;
  if (aliased({{o, qbytes}, {workspace, L.total}},
              {{q, qbytes}, {k, kvbytes}, {v, kvbytes}, {cu_seqlens_q, cubytes}, {cu_seqlens_k, cubytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  sage::SeqSpan* spans = at<sage::SeqSpan>(workspace, L.spans);
  int32_t* qp_owner = at<int32_t>(workspace, L.qp_owner);
  st = fp4_varlen_quant_launch(d, q, k, v, cu_seqlens_q, cu_seqlens_k, sm_scale, spans, qp_owner,
                               at<uint8_t>(workspace, L.q_codes), at<uint8_t>(workspace, L.q_scale),
                               at<uint8_t>(workspace, L.k_codes), at<uint8_t>(workspace, L.k_scale),
                               at<float>(workspace, L.k_mean), at<uint8_t>(workspace, L.v_codes),
                               at<uint8_t>(workspace, L.v_scale), at<double>(workspace, L.ksum), true, has_k,
                               hs);
  if (st != SAGE_OK) return st;
  sage::Fp4AttnArgs a{};
  a.q4 = at<uint8_t>(workspace, L.q_codes);
  a.q_sc = at<uint8_t>(workspace, L.q_scale);
  a.k4 = at<uint8_t>(workspace, L.k_codes);
  a.k_sc = at<uint8_t>(workspace, L.k_scale);
  a.v4 = at<uint8_t>(workspace, L.v_codes);
  a.v_sc = at<uint8_t>(workspace, L.v_scale);
  a.o = o;
  a.ogeo = packed_geom(d.Hq, d.D);
  a.B = int(d.B), a.Hq = int(d.Hq), a.Hkv = int(d.Hkv), a.Nq = int(d.max_q), a.Nk = int(d.max_k), a.D = int(d.D);
  a.n_pad = int(d.n_pad);
  a.causal = is_causal != 0;
  a.bf16 = d.bf16;
  a.seq = spans;
  a.total_q = int(d.total_q);
  a.total_k = int(d.total_k);
  a.qp_owner = qp_owner;
  a.n_owner = int(sage::varlen_qpair_bound(d.total_q, d.B));
  return from_hip(sage::launch_attn_fp4(a, hs));
}

size_t sage_quant_fp4_varlen_workspace_bytes(const sage_varlen_shape* s) {
  VDims d;
  return check_fp4_varlen_shape(s, &d) == SAGE_OK ? fp4_varlen_layout_for(d, true).total : 0;
}

sage_status sage_quant_fp4_varlen(const sage_varlen_shape* s, const void* q, const void* k, const void* v,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, float sm_scale,
                                  uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
                                  float* k_mean, uint8_t* v_codes, uint8_t* v_scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  VDims d;
  sage_status st = check_fp4_varlen_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID_ARGUMENT;
  if (d.B == 0) return SAGE_OK;
  const bool has_q = d.total_q > 0 && d.max_q > 0, has_k = d.total_k > 0 && d.max_k > 0;
  if (!cu_seqlens_q || !cu_seqlens_k || !workspace) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_q && (!q || !q_codes || !q_scale)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!k || !v || !k_codes || !k_scale || !k_mean || !v_codes || !v_scale)) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(workspace, 256)) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_q && (!aligned(q, 16) || !aligned(q_codes, 16) || !aligned(q_scale, 4))) return SAGE_ERR_INVALID_ARGUMENT;
  if (has_k && (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, 16) || !aligned(k_scale, 4) ||
                !aligned(k_mean, 4) || !aligned(v_codes, 16) || !aligned(v_scale, 16)))
    return SAGE_ERR_INVALID_ARGUMENT;
  const Fp4VLayout L = fp4_varlen_layout_for(d, true);
  if (workspace_bytes < L.total) return SAGE_ERR_WORKSPACE;
  const Fp4VSizes z = fp4_varlen_sizes(d);
  const size_t qin = has_q ? size_t(d.Hq * d.total_q * d.D) * 2 : 0, kin = has_k ? size_t(d.Hkv * d.total_k * d.D) * 2 : 0;
  const size_t cubytes = size_t(d.B + 1) * 4;
  if (aliased({{q_codes, has_q ? z.q_codes : 0}, {q_scale, has_q ? z.q_scale : 0}, {k_codes, has_k ? z.k_codes : 0},
               {k_scale, has_k ? z.k_scale : 0}, {k_mean, has_k ? z.k_mean : 0}, {v_codes, has_k ? z.v_codes : 0},
               {v_scale, has_k ? z.v_scale : 0}, {workspace, L.total}},
              {{q, qin}, {k, kin}, {v, kin}, {cu_seqlens_q, cubytes}, {cu_seqlens_k, cubytes}}))
    return SAGE_ERR_INVALID_ARGUMENT;
  return fp4_varlen_quant_launch(d, q, k, v, cu_seqlens_q, cu_seqlens_k, sm_scale,
                                 at<sage::SeqSpan>(workspace, L.spans), at<int32_t>(workspace, L.qp_owner), q_codes,
                                 q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, at<double>(workspace, L.ksum),
                                 has_q, has_k, static_cast<hipStream_t>(stream));
}

sage_status sage_debug_qk_i32(const sage_shape* s, const int8_t* q_codes, const int8_t* k_codes, int32_t* s_out,
                              void* stream) {
  Dims d;
  sage_status st = check_shape(s, &d);
  if (st != SAGE_OK) return st;
  if (d.B == 0 || d.Nq == 0 || d.Nk == 0) return SAGE_OK;
  if (!q_codes || !k_codes || !s_out) return SAGE_ERR_INVALID_ARGUMENT;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(s_out, 4)) return SAGE_ERR_INVALID_ARGUMENT;
  {
    // s_out holds B*Hq*Nq*Nk int32 (saturated: the product can pass 2^64 bytes)
    const int64_t rows = d.B * d.Hq * d.Nq;
    const size_t sbytes = rows > int64_t(SIZE_MAX / 4) / d.Nk ? SIZE_MAX : size_t(rows * d.Nk) * 4;
    if (aliased({{s_out, sbytes}}, {{q_codes, size_t(rows * d.D)}, {k_codes, size_t(d.B * d.Hkv * d.Nk * d.D)}}))
      return SAGE_ERR_INVALID_ARGUMENT;
  }
  sage::DebugQKArgs a{};
  a.q8 = q_codes;
  a.k8 = k_codes;
  a.s_out = s_out;
  a.B = int(d.B), a.Hq = int(d.Hq), a.Hkv = int(d.Hkv), a.Nq = int(d.Nq), a.Nk = int(d.Nk), a.D = int(d.D);
  return from_hip(sage::launch_debug_qk(a, static_cast<hipStream_t>(stream)));
}

const char* sage_status_string(sage_status st) {
  // A C caller may pass any int; read its bits as one, since a value outside
  // the enumerators is not a valid value of the C++ enum type.
  int32_t v;
  static_assert(sizeof(st) == sizeof(v), "sage_status is passed as an int");
  std::memcpy(&v, &st, sizeof v);
  switch (v) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARGUMENT: return "SAGE_ERR_INVALID_ARGUMENT: invalid pointer, size, alignment or enum";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED: head_dim must be 64 or 128; causal needs seq_q == seq_k";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE: workspace smaller than the size query reports";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP: the HIP runtime rejected a launch";
  }
  return "unknown sage_status";
}

}  // extern "C"
